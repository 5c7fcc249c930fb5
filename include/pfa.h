/*
 * pfa.h -- packed variable-length attention for AMD Instinct MI355X (gfx950): the forward,
 * its variants (separate query/key tables, fused QKV input with RoPE, block-sparse tile
 * lists, FP8 P.V), the (O, LSE) merge and the backward.
 *
 * Several images' patch tokens are concatenated into one sequence and an int32 prefix
 * table cu_seqlens = [0, len0, len0+len1, ...] tells which rows belong to which image
 * (Mage-Flow page, hankli.space, section "原生分辨率序列打包": the packed_attention
 * listing, q/k/v shaped [total_tokens, num_heads, head_dim], cu_seqlens of shape (B+1,)
 * int32, the varlen call with causal=False).  Tokens of different images never attend
 * to each other: the attention matrix is block-diagonal (same page, the sentence after
 * that listing).  The kernel tiles Q, K and V, keeps a running row maximum and
 * normaliser, accumulates the output block by block and writes only the final result
 * (lmnt.cn GigaPath-Flash page, section 3.2), which in exact arithmetic equals
 *
 *     O[i,h,:]  = sum_j exp(s_ij - M_i) v[j,h,:] / sum_j exp(s_ij - M_i)
 *     LSE[h,i]  = M_i + ln sum_j exp(s_ij - M_i),   s_ij = scale * q[i,h,:].k[j,h,:]
 *
 * over the keys j of the query's own segment, M_i = max_j s_ij.
 *
 * Every function returns PFA_OK (0) or a negative pfa_status; nothing is thrown across
 * this interface, and nothing is launched when an argument check fails.
 */
#ifndef PFA_H_
#define PFA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PFA_API __attribute__((visibility("default")))

typedef enum pfa_status {
  PFA_OK = 0,
  PFA_ERR_NULL = -1,          /* a required pointer is NULL                              */
  PFA_ERR_NUM_SEQS = -2,      /* num_seqs < 1                                            */
  PFA_ERR_HEADS = -3,         /* heads < 1                                               */
  PFA_ERR_MAX_SEQLEN = -4,    /* max_seqlen < 1                                          */
  PFA_ERR_HEAD_DIM = -5,      /* head_dim is not 64 or 128                               */
  PFA_ERR_SCALE = -6,         /* scale is not finite and > 0                             */
  PFA_ERR_ALIAS = -7,         /* out or lse is the same buffer as an input               */
  PFA_ERR_CU_SEQLENS = -8,    /* host validator: malformed cu_seqlens table              */
  PFA_ERR_DEVICE = -9,        /* no usable device, or a device query failed              */
  PFA_ERR_LAUNCH = -10,       /* the kernel launch reported an error                     */
  PFA_ERR_SIZE = -11,         /* a row (heads * head_dim, 3x that for a fused input) over
                                 2^23 elements, or more than 2^31 - 1 work slots or rows */
  PFA_ERR_ALIGN = -12,        /* a buffer that must be 16-byte aligned is not            */
  PFA_ERR_LAYOUT = -13        /* block-sparse layout: bad layout_heads or nnz; from the
                                 host validator also bad row pointers or block indices,
                                 a repeated block, or a query block with no keys         */
} pfa_status;

/* Block-sparse layouts list key blocks of PFA_SPARSE_BLOCK_K keys per query block of
 * PFA_SPARSE_BLOCK_Q rows, both counted from the start of the segment; segments of a
 * block-sparse call hold at most PFA_SPARSE_MAX_SEQLEN tokens. */
#define PFA_SPARSE_BLOCK_Q 256
#define PFA_SPARSE_BLOCK_K 64
#define PFA_SPARSE_MAX_SEQLEN 65536

/*
 * pfa_varlen_fwd -- packed, non-causal, block-diagonal attention forward.
 *
 * q, k, v     device pointers, bf16, contiguous [T, heads, head_dim]: row t, head h starts
 *             at element (t*heads + h)*head_dim.  T = cu_seqlens[num_seqs] is known only on
 *             the device; this call never reads the table on the host.  Read only.
 * cu_seqlens  device pointer, int32 [num_seqs + 1]: segment s owns rows
 *             [cu_seqlens[s], cu_seqlens[s+1]).  The same table serves queries and keys.
 * num_seqs    number of segments (>= 1).  Zero-length segments are legal and do nothing.
 * max_seqlen  an upper bound on every segment length (>= 1); sizes the launch and picks the
 *             kernel: at most 256 (head_dim 128) or 128 (head_dim 64), each segment's K
 *             and V are loaded into LDS whole (the resident kernel of pfa_varlen_fwd_qk),
 *             above it they stream in 64-key stages.  Both give bitwise equal results.
 * heads       attention heads (>= 1); q, k and v all have this many (no grouped heads).
 * head_dim    64 or 128.
 * scale       factor on q.k, finite and > 0 (1/sqrt(head_dim) in the usual definition).
 * out         device pointer, bf16 [T, heads, head_dim], written (round to nearest even).
 * lse         device pointer, fp32 [heads, T], natural-log sum-exp of the scaled scores;
 *             may be NULL when the caller does not need it.
 * stream      HIP stream to enqueue on (0 = the null stream).  The call returns without
 *             waiting; completion is the caller's to await.
 *
 * Ownership: the caller allocates and owns every buffer; out and lse must not overlap
 * q, k, v or cu_seqlens.  The library allocates no device memory and keeps no state
 * beyond a per-device cache of launch limits, so calls may run concurrently on
 * different streams.
 *
 * Preconditions not checked here (checking them would need a device-to-host copy of the
 * table): cu_seqlens[0] == 0, the table is non-decreasing, every length <= max_seqlen,
 * and the buffers hold T rows.  Use pfa_check_cu_seqlens on a host copy to verify them.
 * If they are violated the result is undefined, but the kernel still writes no row
 * outside [0, cu_seqlens[num_seqs]).
 *
 * Results are deterministic: each output row and LSE entry is produced by exactly one
 * workgroup in a fixed order, with no atomics.
 */
PFA_API int pfa_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                           int num_seqs, int max_seqlen, int heads, int head_dim, float scale,
                           void* out, float* lse, hipStream_t stream);

/*
 * pfa_varlen_fwd_qk -- the same forward with separate query and key segment tables.
 *
 * The varlen call of the Mage-Flow packed_attention listing takes cu_seqlens_q and
 * cu_seqlens_k (and max_seqlen_q / max_seqlen_k) as separate arguments; pfa_varlen_fwd
 * is the case where both are one table.  With different tables, the queries of segment s
 * are rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) of q and attend exactly the keys
 * [cu_seqlens_k[s], cu_seqlens_k[s+1]) of k and v: the cross-attention of the xxmr.cn
 * editing-network article (section 3.1: queries from the draft features, keys and values
 * from the condition or edit sequence; section 4.1: those sequences are much shorter than
 * the query sequence).
 *
 * q, out        bf16 [Tq, heads, head_dim], Tq = cu_seqlens_q[num_seqs].
 * k, v          bf16 [Tk, heads, head_dim], Tk = cu_seqlens_k[num_seqs].
 * cu_seqlens_q, cu_seqlens_k   device int32 [num_seqs + 1]; passing the same pointer for
 *               both selects the self-attention instantiation of the streaming kernel
 *               (when max_seqlen_k is above the resident bound below).
 * max_seqlen_q  bound on every query segment length (>= 1); sizes the launch.
 * max_seqlen_k  bound on every key segment length (>= 1).  At most 256 (head_dim 128) or
 *               128 (head_dim 64) selects a kernel that holds each (segment, head)'s K and V
 *               in LDS for all of its query tiles; above it K/V stream in 64-key stages.
 *               Both give bitwise equal results.  A key segment longer than this bound
 *               breaks the precondition below: the resident kernel then reads only its
 *               first 256 (128) keys, and still reads and writes no row out of range.
 * lse           fp32 [heads, Tq] or NULL.
 * Everything else, ownership and errors as for pfa_varlen_fwd.  A segment with queries
 * but no keys has no softmax; its rows get O = 0 and LSE = -inf.  Both tables must
 * satisfy the preconditions of pfa_varlen_fwd (check each with pfa_check_cu_seqlens).
 */
PFA_API int pfa_varlen_fwd_qk(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int num_seqs, int max_seqlen_q, int max_seqlen_k, int heads,
                              int head_dim, float scale, void* out, float* lse,
                              hipStream_t stream);

/*
 * pfa_varlen_fwd_qkv -- the self-attention forward read straight from a fused projection
 * output, with optional rotary position embedding of q and k.
 *
 * The DiT block of the Mage-Flow page (section on its fusion opportunities) computes q, k
 * and v with one merged W_qkv projection, splits its output into three along the feature
 * axis (chunk(3, dim=-1)), applies RoPE, then attention.  This call takes that output as
 * it is: q, k and v are read through a row stride of 3 * heads * head_dim, with no copy
 * into separate tensors.  The pages do not fix the RoPE variant; this is the rotate-half
 * pairing: for i < head_dim / 2, features (x_i, x_{i + head_dim/2}) of token t, every
 * head, become
 *     (x_i cos[t][i] - x_{i+d/2} sin[t][i],  x_{i+d/2} cos[t][i] + x_i sin[t][i]),
 * evaluated in fp32 and rounded to bf16 (nearest even) before the attention of
 * pfa_varlen_fwd.  Per-token tables cover any position scheme (1-D, axial 2-D or 3-D):
 * the caller writes each token's angles.
 *
 * qkv         device bf16 [T, 3, heads, head_dim] (row t: q, then k, then v, each
 *             heads * head_dim values, head-major); 16-byte aligned.  Read only.
 * rope_cos, rope_sin   device fp32 [T, head_dim / 2], 16-byte aligned, or both NULL for
 *             no rotation.
 * k_rot       with tables: device bf16 [T, heads, head_dim] workspace, 16-byte aligned,
 *             owned by the caller; on return (stream-ordered) it holds the rotated keys.
 *             Keys are rotated there by one pass before the attention kernel, which
 *             re-reads every key once per 256-query tile; queries are rotated in
 *             registers as they are loaded.  Ignored (may be NULL) without tables.
 * out, lse    as for pfa_varlen_fwd (out 16-byte aligned).
 * cu_seqlens, num_seqs, max_seqlen, heads, head_dim, scale, stream: as for pfa_varlen_fwd.
 * Errors: as for pfa_varlen_fwd, plus PFA_ERR_NULL for one table without the other or
 * tables without k_rot, PFA_ERR_ALIAS when out, lse or k_rot is an input or two of them
 * coincide, PFA_ERR_ALIGN, and PFA_ERR_SIZE when 3 * heads * head_dim exceeds 2^23.
 */
PFA_API int pfa_varlen_fwd_qkv(const void* qkv, const float* rope_cos, const float* rope_sin,
                               const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                               int heads, int head_dim, float scale, void* out, float* lse,
                               void* k_rot, hipStream_t stream);

/*
 * pfa_varlen_fwd_blocksparse -- the packed self-attention forward restricted to listed
 * key blocks.
 *
 * The SparseAttn article (jefxiong.cn, "AIGC 基本功｜视频稀疏注意力的误差与布局") defines a
 * sparse row as the softmax restricted to the row's retained key set and renormalised over
 * it (section 3.1). It notes that a kernel saves work only when it skips whole blocks it
 * knows in advance (sections 04 and 06), and that sliding-tile attention lets each query
 * tile share one set of key tiles (section 05). Here the retained set of a query is
 * chosen at block granularity. Query i of segment s (rows [a, a + L)) lies in query block
 * (i - a) / PFA_SPARSE_BLOCK_Q. It attends the keys j of its own segment whose key block
 * (j - a) / PFA_SPARSE_BLOCK_K is listed for (s, its head, its query block):
 *     O[i,h,:] = sum_{j listed} exp(s_ij - M_i) v[j,h,:] / sum_{j listed} exp(s_ij - M_i),
 *     LSE[h,i] = M_i + ln sum_{j listed} exp(s_ij - M_i),   M_i = max over the listed keys.
 * Listed blocks are computed whole and unlisted ones are skipped (never loaded).
 *
 * kv_ptr, kv_idx  device int32 CSR of the lists. qt_max = ceil(max_seqlen /
 *             PFA_SPARSE_BLOCK_Q); row r = (s * layout_heads + hl) * qt_max + qb holds the
 *             key-block indices kv_idx[kv_ptr[r] .. kv_ptr[r+1]) of segment s, layout head
 *             hl and query block qb. kv_ptr has num_seqs * layout_heads * qt_max + 1 entries
 *             and kv_idx has nnz (kv_idx may be NULL when nnz is 0). Rows of query blocks a
 *             segment does not have are ignored. Indices outside the segment's key blocks
 *             are skipped. The order of a list is free. A repeated index counts its keys
 *             twice, and the validator rejects it.
 * layout_heads 1 (every head uses the same lists, hl = 0) or heads (hl = h).
 * Everything else as for pfa_varlen_fwd. max_seqlen must not exceed PFA_SPARSE_MAX_SEQLEN
 * (PFA_ERR_SIZE).
 *
 * A query block whose list retains no key has no softmax. Its rows get O = 0 and
 * LSE = -inf. The article treats such rows as invalid input, and the validator rejects
 * them. Checked here: NULL pointers, the scalars, layout_heads and nnz (PFA_ERR_LAYOUT),
 * aliasing of out or lse with an input. The row pointers are clamped to [0, nnz] on the
 * device, so a malformed table never makes the kernel read outside kv_ptr's rows or
 * kv_idx's nnz entries.
 */
PFA_API int pfa_varlen_fwd_blocksparse(const void* q, const void* k, const void* v,
                                       const int32_t* cu_seqlens, int num_seqs, int max_seqlen,
                                       int heads, int head_dim, float scale,
                                       const int32_t* kv_ptr, const int32_t* kv_idx, int nnz,
                                       int layout_heads, void* out, float* lse,
                                       hipStream_t stream);

/*
 * pfa_check_block_layout -- host validator for a block-sparse layout (host copies of the
 * tables). It checks cu_seqlens as pfa_check_cu_seqlens does, then: kv_ptr[0] = 0,
 * non-decreasing, kv_ptr[rows] = nnz; every index within its segment's key blocks; no
 * index repeated in a row; no existing query block with an empty list (SparseAttn article,
 * section 09: rows with no retained key are rejected); and rows of query blocks a segment
 * does not have are empty. Returns PFA_OK or the first failing code (PFA_ERR_LAYOUT for the
 * layout itself).
 */
PFA_API int pfa_check_block_layout(const int32_t* cu_host, int num_seqs, int max_seqlen,
                                   int heads, int layout_heads, const int32_t* kv_ptr_host,
                                   const int32_t* kv_idx_host, int nnz);

/*
 * pfa_quantize_v_fp8 -- V in e4m3 for pfa_varlen_fwd_fp8pv.
 *
 * The FPS Attention slides (tool.lu deck "[极致]加速多模态生成的算法设计与系统挑战",
 * slides 35-38) quantise V per channel for an FP8 attention that dequantises as it goes. The
 * slides fix no format or scale rule. Here every (segment, head, channel) gets a
 * power-of-two scale 2^e: e is the smallest integer with max_t |V[t,h,c]| * 2^-e <= 448
 * (the largest OCP e4m3 value), not below -126, and e = 0 for an all-zero channel. The code
 * of V[t,h,c] is V * 2^-e rounded to e4m3, to nearest even. Scaling by a power of two is
 * exact, and a segment's scales depend on its own tokens only, so packing does not couple
 * images.
 *
 * v         device bf16 [T, heads, head_dim], 16-byte aligned, finite.
 * v8        device uint8 [T, heads, head_dim] e4m3 codes, 8-byte aligned (written).
 * v_scale   device fp32 [num_seqs, heads, head_dim] (written): the scales 2^e. During the
 *           call it holds the per-channel maxima.
 * Four kernel launches on stream (HBM-bound). Errors as for pfa_varlen_fwd, plus
 * PFA_ERR_ALIAS, PFA_ERR_ALIGN, and PFA_ERR_SIZE when num_seqs * heads * head_dim exceeds
 * 2^31 - 1.
 */
PFA_API int pfa_quantize_v_fp8(const void* v, const int32_t* cu_seqlens, int num_seqs, int heads,
                               int head_dim, void* v8, float* v_scale, hipStream_t stream);

/*
 * pfa_varlen_fwd_fp8pv -- the packed self-attention forward with P.V in FP8.
 *
 * The same blocked online softmax as pfa_varlen_fwd, with q.k in bf16. For every 64-key
 * block, the weights w = 2^8 * exp(s - m) (m the running row maximum, so w <= 2^8: P
 * quantised per tensor with the fixed scale 2^8) are rounded to e4m3. They multiply the
 * e4m3 codes of V on the FP8 matrix cores, with fp32 accumulation. The row sum l adds
 * the unrounded weights and normalises the output:
 *     O[i,h,c] = v_scale[s,h,c] * sum_j e4m3(w_ij) v8[j,h,c] / l_i,
 *     LSE[h,i] = m_i - 8 ln 2 + ln l_i  (as in pfa_varlen_fwd, from unrounded weights).
 * Each weight's rounding is at most 2^-4 of it (2^-10 absolute below 2^-6). Against exact
 * attention on the dequantised V, O therefore errs by at most
 * sum_j (2^-4 p_ij + 2^-18) |V_j| / sum_j p_ij, plus the bf16 rounding of O.
 *
 * q, k      bf16 [T, heads, head_dim] as for pfa_varlen_fwd.
 * v8, v_scale  as written by pfa_quantize_v_fp8 (both 16-byte aligned).
 * Everything else, ownership and errors as for pfa_varlen_fwd, plus PFA_ERR_ALIGN.
 */
PFA_API int pfa_varlen_fwd_fp8pv(const void* q, const void* k, const void* v8, const float* v_scale,
                                 const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int heads,
                                 int head_dim, float scale, void* out, float* lse,
                                 hipStream_t stream);

/*
 * pfa_varlen_fwd_blocksparse_fp8pv -- FPS Attention: block-sparse tile lists with P.V in FP8.
 *
 * The FPS Attention slides (tool.lu deck, slides 35-38) combine sliding-tile sparsity with
 * FP8 attention. This is pfa_varlen_fwd_blocksparse (the same CSR lists, block sizes,
 * limits and empty-row convention) with the FP8 arithmetic of pfa_varlen_fwd_fp8pv (V
 * from pfa_quantize_v_fp8, e4m3 weights scaled by 2^8, O normalised by the unrounded
 * weights). The running maximum visits the listed blocks in list order. Arguments and
 * errors are the union of the two calls'.
 */
PFA_API int pfa_varlen_fwd_blocksparse_fp8pv(const void* q, const void* k, const void* v8,
                                             const float* v_scale, const int32_t* cu_seqlens,
                                             int num_seqs, int max_seqlen, int heads,
                                             int head_dim, float scale, const int32_t* kv_ptr,
                                             const int32_t* kv_idx, int nnz, int layout_heads,
                                             void* out, float* lse, hipStream_t stream);

/*
 * pfa_attn_merge -- combine two results for the same queries over disjoint key sets.
 *
 * If (o_a, lse_a) is attention over key set A and (o_b, lse_b) over key set B, the
 * attention over A and B together has partition sum exp(lse_a) + exp(lse_b) and output
 *     out = (exp(lse_a) o_a + exp(lse_b) o_b) / (exp(lse_a) + exp(lse_b)),
 *     lse = ln(exp(lse_a) + exp(lse_b)),
 * the identity behind the blocked running-max / normaliser update of the GigaPath-Flash
 * page (section 3.2), applied to two finished blocks.  It joins per-block results of
 * pfa_varlen_fwd_qk (e.g. key sets split across devices or passes).  A side with
 * lse = -inf (no keys) contributes nothing; two such sides give out = 0, lse = -inf.
 *
 * o_a, o_b, out  device bf16 [total, heads, head_dim]; out may be o_a or o_b (in place).
 * lse_a, lse_b   device fp32 [heads, total]; lse may be lse_a or lse_b, or NULL.
 * total          rows (>= 0; 0 does nothing).
 * Arithmetic in fp32, output rounded to nearest even.  Returns PFA_OK, PFA_ERR_NULL,
 * PFA_ERR_SIZE, PFA_ERR_HEADS, PFA_ERR_HEAD_DIM (64 or 128), PFA_ERR_ALIAS (an O buffer
 * shared with an LSE buffer) or PFA_ERR_LAUNCH.  Enqueued on stream; returns at once.
 */
PFA_API int pfa_attn_merge(const void* o_a, const float* lse_a, const void* o_b,
                           const float* lse_b, int64_t total, int heads, int head_dim,
                           void* out, float* lse, hipStream_t stream);

/*
 * pfa_varlen_bwd -- gradients of pfa_varlen_fwd (self-attention, one segment table).
 *
 * The pages train with this packed path (Mage-Flow page: the gains of packing are
 * training throughput) but print no gradient formulas; the operation is the chain rule of
 * the forward definition above.  For upstream gradient dO of O, per segment and head,
 * with P the softmax rows (recomputed from lse) and s_ij = scale q_i.k_j:
 *     dV = P^T dO,   dP = dO V^T,   delta_i = dO_i . O_i (= sum_j P_ij dP_ij),
 *     dS = P * (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q.
 *
 * q, k, v, out, dout  device bf16 [T, heads, head_dim] (out: the forward's output).
 * lse         device fp32 [heads, T]: the forward's LSE (natural log).  Required.
 * cu_seqlens, num_seqs, max_seqlen, heads, head_dim, scale: as for pfa_varlen_fwd.
 * dq, dk, dv  device bf16 [T, heads, head_dim], written (round to nearest even).
 * workspace   device fp32 [2, heads, T], written: -lse*log2(e) and delta.  The caller
 *             owns it; its contents after the call are not part of the interface.
 * Ownership and errors as for pfa_varlen_fwd; PFA_ERR_ALIAS if an output (dq, dk, dv,
 * workspace) is an input or another output.  Two kernels are enqueued on stream (the dQ
 * pass, which also writes the row statistics to workspace, then the dK/dV pass, which
 * reads them); no atomics, so results are deterministic.
 */
PFA_API int pfa_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, const int32_t* cu_seqlens,
                           int num_seqs, int max_seqlen, int heads, int head_dim, float scale,
                           void* dq, void* dk, void* dv, float* workspace, hipStream_t stream);

/* Capacity, in fp32 values, of the device array that holds the row statistics of
 * pfa_varlen_bwd_noalloc: 2 * heads * T of them must fit (heads * T <= 4,194,304). */
#define PFA_BWD_SCRATCH_FLOATS (1 << 23)

/*
 * pfa_varlen_bwd_noalloc -- pfa_varlen_bwd for callers that cannot allocate device memory
 * (code under graph capture, tight serving or training loops, harnesses that forbid
 * allocation): the same gradients from the same two kernels, with the 2 * heads * T fp32
 * row statistics kept in a library-held device array instead of a caller workspace.
 *
 * The array holds PFA_BWD_SCRATCH_FLOATS values (32 MiB), one copy per device the
 * library runs on, allocated with the library's GPU code and held until the process ends.
 * Its device address is looked up once per device, on the first call with that device
 * current.  This call allocates and frees nothing.
 *
 * total_tokens  T = cu_seqlens[num_seqs], which the host cannot read without a copy; it
 *               sizes the check 2 * heads * total_tokens <= PFA_BWD_SCRATCH_FLOATS
 *               (PFA_ERR_SIZE otherwise).  If the table's last entry differs, the result is
 *               undefined, but no access leaves the array: the kernels do nothing when the
 *               table's T exceeds the array's capacity.
 * Every other argument, the ownership rules and the errors are those of pfa_varlen_bwd.
 *
 * All calls on one device share that device's array and each call overwrites it, so two
 * calls that overlap in time on one device (different streams, or several host threads)
 * race and their results are undefined.  Calls on one stream are ordered and safe.
 */
PFA_API int pfa_varlen_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* lse, const int32_t* cu_seqlens,
                                   int num_seqs, int max_seqlen, int64_t total_tokens, int heads,
                                   int head_dim, float scale, void* dq, void* dk, void* dv,
                                   hipStream_t stream);

/*
 * pfa_check_cu_seqlens -- host-side validator of a cu_seqlens table (no device calls).
 *
 * cu_host     host pointer to num_seqs + 1 int32 values.
 * num_seqs    >= 1.
 * max_seqlen  the bound that will be passed to pfa_varlen_fwd (>= 1).
 * total_out   if not NULL, receives cu_host[num_seqs] (the packed token count T).
 *
 * Returns PFA_OK when cu_host[0] == 0, the table is non-decreasing and every segment
 * length is <= max_seqlen; PFA_ERR_NULL, PFA_ERR_NUM_SEQS, PFA_ERR_MAX_SEQLEN or
 * PFA_ERR_CU_SEQLENS otherwise.
 */
PFA_API int pfa_check_cu_seqlens(const int32_t* cu_host, int num_seqs, int max_seqlen,
                                 int64_t* total_out);

/* pfa_status_string -- static text for a status code (never NULL). */
PFA_API const char* pfa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PFA_H_ */
