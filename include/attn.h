/*
 * attn.h — C ABI of the exact-attention library for AMD Instinct MI355X
 * (gfx950).  Build: libattn.so (hipcc --offload-arch=gfx950).
 *
 * The operation is exact softmax attention, computed tile by tile without
 * ever storing the N x N score matrix:
 *
 *   O = softmax(scale * Q K^T [+ causal mask]) V
 *
 * (FlashAttention pages: the formula at the top of "FlashAttention：让精确注意力
 * 服从内存层次" (wineandchord.com); the tiling and online-softmax passages and
 * the conceptual forward pass of the "FlashAttention" paper story
 * (ai.tomabc.com)).  Alongside O the forward stores one statistic per query
 * row, the natural-log logsumexp of that row's scaled scores; the backward
 * recomputes the probabilities from it (the recomputation paragraph of the
 * same paper story) instead of reading an N x N matrix.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, contiguous, row-major (the *_strided entry points
 *    take element strides instead):
 *        Q, O, dQ, dO : [B, Hq,  N, d]
 *        K, V, dK, dV : [B, Hkv, N, d]
 *        LSE          : [B, Hq,  N]      (fp32, natural log)
 *    Query head h reads key/value head h / (Hq / Hkv) (grouped-query
 *    attention; Hq must be a multiple of Hkv; Hq == Hkv is plain multi-head).
 *  - Causal mask (causal = 1): key j is visible to query i iff j <= i.
 *  - scale multiplies Q K^T; any finite value is accepted (callers usually
 *    pass 1/sqrt(d)).
 *  - Every pointer is a DEVICE pointer on the current HIP device, 16-byte
 *    aligned.  The caller owns and allocates all memory (including the
 *    backward workspace); the library allocates nothing, keeps no state
 *    between calls other than a per-device architecture check, and is safe
 *    to call from several host threads on different streams.
 *  - Outputs must not overlap inputs or each other.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream).  The call returns once the kernels are launched;
 *    it never synchronises, unless the environment variable ATTN_DEBUG is
 *    set (to anything but "" or "0"; read at every call): then every entry
 *    point synchronises `stream` after its launches and returns
 *    ATTN_ERR_HIP if they failed, so a failing kernel is reported by the
 *    call that launched it (debugging only; not under graph capture).
 *  - Sizes: N <= 2^22 and B * Hq <= 2^24, and every launch must fit one
 *    dispatch of fewer than 2^32 work-items: B * Hq * (N rounded up to 128)
 *    * max(8, d / 8) < 2^32 (larger requests return ATTN_ERR_UNSUPPORTED).
 *  - Value range (16-bit paths): the online softmax moves its running row
 *    maximum lazily, only once a row's scores exceed it by more than tau
 *    (base 2; tau = 30 for bf16, 15 for fp16), so probabilities carried in
 *    the fp32 accumulators are at most 2^tau instead of 1.  bf16 outputs are
 *    therefore within range as long as (number of visible keys) * max|V| <
 *    2^98 (about 3e29; a plain online softmax allows up to 3.4e38).  fp16
 *    inputs cannot reach the limit (2^15 * 65504 * 2^22 < 2^128).  The
 *    backward rounds P (at most 1 there) and dS = P * (dP - D) to the input
 *    type for its dV, dK and dQ products (fp32 accumulation): with fp16 it
 *    needs |dO_i . v_j - D_i| < 65504 wherever P_ij is not negligible, else
 *    those gradients overflow; bf16 has fp32's range.
 *  - B == 0 or N == 0 is an empty problem: nothing is launched and ATTN_OK
 *    is returned (pointers may then be NULL).
 *  - Arguments are validated on the host before any HIP call.  On error no
 *    kernel is launched and no output is touched.
 *
 * Supported: dtype ATTN_BF16 or ATTN_F16 (16-bit inputs/outputs, fp32
 * accumulation on the matrix cores, probabilities rounded to the same 16-bit
 * type for the P V product) with d in {64, 128, 256}; dtype ATTN_F32 (fp32
 * throughout, vector ALUs, forward only) with d in {64, 128}.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,        /* bad pointer, size, alignment or overlap */
  ATTN_ERR_UNSUPPORTED = 2,        /* valid request the library does not implement */
  ATTN_ERR_UNSUPPORTED_DEVICE = 3, /* current device is not gfx950 */
  ATTN_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_F16 = 2 } attn_dtype;

/* Version of this ABI; bumped on any incompatible change. */
int attn_abi_version(void);

/*
 * Forward pass.
 *   q    [B,Hq,N,d]  in   (dtype)
 *   k, v [B,Hkv,N,d] in   (dtype)
 *   o    [B,Hq,N,d]  out  (dtype)  softmax(scale*q k^T [+mask]) v, per head
 *   lse  [B,Hq,N]    out  (fp32)   ln sum_j exp(scale * q_i . k_j) over the
 *                                  visible keys j of row i
 * Tiling: each workgroup holds a block of query rows on chip while key/value
 * tiles stream through LDS; the running row maximum and normaliser rescale
 * the on-chip accumulator (online softmax), so only O and LSE reach memory.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     attn_dtype dtype, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for this problem (a multiple of
 * 256).  0 for an empty problem.  Returns (size_t)-1 for arguments attn_bwd
 * would reject.  The workspace holds the row statistics (8 * B * Hq * (N
 * rounded up to 64) bytes, rounded up to 256) and, for grouped-query problems
 * whose grid of key blocks x (batch, kv head) would leave the device mostly
 * idle, fp32 partial sums of dK and dV after them: the dK/dV stage then
 * splits each group's query heads over S workgroups per key block and merges
 * their sums in a fixed order (2 * S * B * Hkv * N * d * 4 bytes, rounded up
 * to 256; S is chosen from the shape, at most Hq / Hkv).
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d, attn_dtype dtype);

/*
 * Backward pass with recomputation.
 *   q, k, v, o, lse  in   as produced for / by attn_fwd with the same
 *                         B, Hq, Hkv, N, d, causal, scale, dtype
 *   dout [B,Hq,N,d]  in   upstream gradient dL/dO (dtype)
 *   dq   [B,Hq,N,d]  out  dL/dQ (dtype)
 *   dk, dv [B,Hkv,N,d] out dL/dK, dL/dV (dtype), summed over the query heads
 *                         that share each key/value head
 *   workspace        scratch of attn_bwd_workspace_bytes(...) bytes, owned by
 *                    the caller, contents need not be initialised; it must
 *                    stay allocated until the launched work completes.
 * The softmax probabilities are recomputed tile by tile from q, k and lse;
 * no N x N matrix is read or written.  Deterministic (no atomics).
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     void* workspace, int B, int Hq, int Hkv, int N, int d, int causal,
                     float scale, attn_dtype dtype, void* stream);

/*
 * attn_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (without `workspace`), validation and results as attn_bwd, bit for
 * bit: the same kernels with the same launch plan, the workspace placed in a
 * scratch array of ATTN_NOALLOC_SCRATCH_BYTES that the library keeps in
 * static device memory on every device it runs on until the process ends
 * (its address is looked up on the first call on each device).  Nothing is
 * allocated or freed.
 *   - Problems whose attn_bwd_workspace_bytes(...) exceeds
 *     ATTN_NOALLOC_SCRATCH_BYTES return ATTN_ERR_UNSUPPORTED (for example
 *     B * Hq * (N rounded up to 64) > 4M rows, or a grouped-query split whose
 *     partial sums do not fit).
 *   - Every call on a device shares that device's scratch.  Calls whose work
 *     overlaps in time on one device race on it and give wrong results:
 *     issue them on one stream, or order them with events.  The scratch keeps
 *     the last call's contents; no call depends on them (each reads only what
 *     it wrote first).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
attn_status attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                             attn_dtype dtype, void* stream);

/*
 * The backward as three separate stages on one stream, exposed so a caller
 * can schedule or time them separately; calling them in this order with the
 * same arguments gives exactly attn_bwd's results (bit for bit).  attn_bwd
 * itself launches two kernels: the dQ stage in a variant that also computes
 * and stores the statistics below, then the dK/dV stage.
 *
 * `stats` is the backward workspace (attn_bwd_workspace_bytes bytes, caller
 * owned).  It starts with per (batch, query head) two fp32 rows of Np = N
 * rounded up to 64 entries, [B*Hq][2][Np]: -D_i = -(dO_i . O_i) and
 * LSE_i * log2(e), zero in the padding.  attn_bwd_preprocess writes them; the
 * other two stages read them.  attn_bwd_dkdv also writes the workspace's
 * partial-sum region after them when it splits query heads (see
 * attn_bwd_workspace_bytes), so it takes `stats` as writable and needs the
 * whole workspace; the other stages need only the statistics.
 *
 *   attn_bwd_preprocess: the row statistics from O, dO and LSE.
 *   attn_bwd_dkdv:       dK, dV, recomputing P and dP tile by tile from q, k
 *                        and the statistics; dK/dV of a key/value head are
 *                        summed over its query heads on chip.
 *   attn_bwd_dq:         dQ, recomputing P and dP the same way.
 * Validation, ownership and error behaviour are those of attn_bwd.
 */
attn_status attn_bwd_preprocess(const void* o, const void* dout, const float* lse, float* stats,
                                int B, int Hq, int N, int d, attn_dtype dtype, void* stream);
attn_status attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                          float* stats, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                          int causal, float scale, attn_dtype dtype, void* stream);
attn_status attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                        const float* stats, void* dq, int B, int Hq, int Hkv, int N, int d,
                        int causal, float scale, attn_dtype dtype, void* stream);

/*
 * The dQ stage fused with the preprocess: dQ as attn_bwd_dq computes it, and
 * the statistics attn_bwd_preprocess would write (bit for bit), computed by
 * the same workgroups from o, dout and lse and written to `stats` (which is
 * an output here; its prior contents are ignored).  attn_bwd is this call
 * followed by attn_bwd_dkdv.  Arguments, validation, ownership and error
 * behaviour are attn_bwd's, with `stats` in place of its workspace.
 */
attn_status attn_bwd_dq_stats(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, float* stats, void* dq, int B,
                              int Hq, int Hkv, int N, int d, int causal, float scale,
                              attn_dtype dtype, void* stream);

/*
 * Split-K/V forward, for few queries against many keys (decoding one token,
 * or appending a short chunk, against a long key/value cache: the decode row
 * of the shape table in "FlashAttention：让精确注意力服从内存层次", section
 * "训练与推理的形状不同", whose first constraint is key/value bandwidth).
 *   q    [B,Hq,Nq,d]  in   (dtype: bf16 or fp16)
 *   k, v [B,Hkv,Nk,d] in   (dtype)
 *   o    [B,Hq,Nq,d]  out  (dtype)
 *   lse  [B,Hq,Nq]    out  (fp32, natural log)
 *   workspace         scratch of attn_fwd_splitkv_workspace_bytes(...) bytes
 *                     with the same shape and num_splits; caller owned,
 *                     contents need not be initialised, must stay allocated
 *                     until the launched work completes.
 * Same operation as attn_fwd, with Nq queries and Nk keys.  The causal mask
 * is aligned to the bottom-right corner: query i sees key j iff
 * j <= i + (Nk - Nq), so the last query sees every key (for Nq == Nk this is
 * attn_fwd's mask).  A query row that sees no key (causal with Nq > Nk, or
 * Nk == 0) gets o = 0 and lse = -inf.
 * The keys of each (batch, key/value head) are cut into num_splits ranges
 * of whole 64-key tiles (num_splits == 0 picks a count from the shape; the
 * count used may be lower than asked, so that no range is empty).  Each range
 * yields a normalised partial output and its logsumexp; a second kernel
 * merges them with the online-softmax merge of ("FlashAttention：让精确注意力
 * 服从内存层次", section "Online softmax"), so the result is the exact
 * attention up to rounding.  The query heads of one key/value head are
 * processed together, so K and V are read once per group.
 * Supported: ATTN_BF16 or ATTN_F16, d in {64, 128, 256}, Nq and Nk <= 2^22,
 * (Hq/Hkv)*Nq <= 2^22, B*Hq <= 2^24 (else ATTN_ERR_UNSUPPORTED).  B == 0 or
 * Nq == 0 is an empty problem (ATTN_OK, nothing launched).  Every other
 * convention is attn_fwd's; pointers must be non-NULL even when Nk == 0.
 */
attn_status attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                             void* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                             int causal, float scale, int num_splits, attn_dtype dtype,
                             void* stream);

/* Number of key ranges attn_fwd_splitkv uses for this shape and request; 0
 * for an empty problem, -1 for arguments it would reject. */
int attn_fwd_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits);

/*
 * attn_fwd_splitkv on tensors of any (batch, head, row) element strides, such
 * as a token-major [B, Nk, Hkv, d] key/value cache.  strides[0..2] address q,
 * strides[3..5] k and v, strides[6..8] o; lse and the workspace stay dense
 * (the workspace is attn_fwd_splitkv_workspace_bytes(...) bytes).  Stride
 * rules as for attn_fwd_strided (with Nq rows for q and o, Nk for k and v),
 * and one head group's query rows must lie within 2^31 bytes of the group's
 * first row: ((Hq/Hkv - 1) * q_h + (Nq - 1) * q_row + d) * 2 < 2^31.  Every
 * other convention is attn_fwd_splitkv's, and with the dense strides the
 * result is attn_fwd_splitkv's bit for bit.
 */
attn_status attn_fwd_splitkv_strided(const void* q, const void* k, const void* v, void* o,
                                     float* lse, void* workspace, const long long* strides, int B,
                                     int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                                     float scale, int num_splits, attn_dtype dtype, void* stream);

/* Bytes of workspace attn_fwd_splitkv needs (a multiple of 256: fp32 partial
 * outputs and logsumexps of every split); 0 for an empty problem,
 * (size_t)-1 for arguments it would reject. */
size_t attn_fwd_splitkv_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                        int num_splits);

/*
 * Block-sparse forward ("FlashAttention" paper story, block-sparse
 * paragraph: a 0/1 mask over the grid of score blocks, whose zero blocks
 * are never loaded or computed).  The blocks are the forward's tiles:
 * ATTN_SPARSE_BLOCK_Q query rows by ATTN_SPARSE_BLOCK_K keys.
 *   q, k, v, o, lse  as attn_fwd (bf16 or fp16), square: N queries and N keys
 *   block_mask  in   DEVICE bytes [mask_heads][ceil(N/128)][ceil(N/64)],
 *                    row-major, any alignment; non-zero = block present.
 *                    mask_heads is 1 (one mask for every head and batch) or
 *                    Hq (one mask per query head, shared by the batch).
 *   workspace        attn_fwd_blocksparse_workspace_bytes(Hq, N, mask_heads)
 *                    bytes, caller owned, need not be initialised; holds the
 *                    compacted list of present blocks of each mask row.
 * Query i of head h sees key j iff
 *   block_mask[h or 0][i / 128][j / 64] != 0  and  (causal == 0 or j <= i).
 * A row that sees no key gets o = 0 and lse = -inf.  Two kernels run on
 * `stream`: the mask compaction, then the forward.  Supported: ATTN_BF16 or
 * ATTN_F16, d in {64, 128, 256}, N <= 2^21 (2^20 at d = 256; else
 * ATTN_ERR_UNSUPPORTED).  mask_heads other than 1 or Hq, or a NULL mask, is
 * ATTN_ERR_INVALID_ARG.  Every other convention is attn_fwd's.
 */
#define ATTN_SPARSE_BLOCK_Q 128
#define ATTN_SPARSE_BLOCK_K 64
attn_status attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const unsigned char* block_mask, int mask_heads, void* workspace,
                                 int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                                 attn_dtype dtype, void* stream);

/*
 * attn_fwd_blocksparse on tensors of any (batch, head, row) element strides:
 * strides[0..8] and their rules as for attn_fwd_strided (the mask, lse and
 * workspace stay dense).  With the dense strides the result is
 * attn_fwd_blocksparse's bit for bit.
 */
attn_status attn_fwd_blocksparse_strided(const void* q, const void* k, const void* v, void* o,
                                         float* lse, const unsigned char* block_mask,
                                         int mask_heads, void* workspace,
                                         const long long* strides, int B, int Hq, int Hkv, int N,
                                         int d, int causal, float scale, attn_dtype dtype,
                                         void* stream);

/* Bytes of workspace attn_fwd_blocksparse needs (a multiple of 256); 0 for
 * N == 0; (size_t)-1 for Hq < 1, N outside [0, 2^21] or mask_heads other
 * than 1 or Hq. */
size_t attn_fwd_blocksparse_workspace_bytes(int Hq, int N, int mask_heads);

/*
 * Packed variable-length forward: nseq sequences of different lengths laid
 * end to end along the token axis (no padding), every token attending only
 * to keys of its own sequence, causally within it if causal = 1.
 *   q, o        [Hq,  T, d]  dtype (bf16 or fp16), token-major within each head
 *   k, v        [Hkv, T, d]  dtype
 *   lse         [Hq,  T]     fp32
 *   cu_seqlens  DEVICE int32 [nseq + 1], 4-byte aligned: sequence s is tokens
 *               [cu_seqlens[s], cu_seqlens[s+1]); the caller guarantees
 *               0 = cu_seqlens[0] <= ... <= cu_seqlens[nseq] = T.  The kernel
 *               clamps every offset into [0, T], so inconsistent offsets
 *               cannot read or write outside the tensors.
 *   max_seqlen  host int, at least the longest sequence (it sizes the grid;
 *               rows of a sequence beyond max_seqlen are not computed),
 *               at most T.
 * Each (sequence, head) is the attention of attn_fwd on that sequence alone;
 * the sequences' key/value ranges are addressed through their own buffer
 * descriptors, so no work is spent on other sequences' keys.  A sequence of
 * length 0 has no rows.  Supported: ATTN_BF16 or ATTN_F16, d in {64, 128,
 * 256}, T <= 2^22,
 * nseq * Hq <= 2^24.  nseq == 0, T == 0 or max_seqlen == 0 launches nothing.
 * Every other convention is attn_fwd's.
 */
attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens, int nseq, int max_seqlen, int Hq, int Hkv,
                            int T, int d, int causal, float scale, attn_dtype dtype,
                            void* stream);

/*
 * Forward on strided tensors: every tensor is addressed as
 *   base + b * stride_b + h * stride_h + i * stride_row + c     (elements)
 * with the d elements of a row contiguous.  strides is a HOST array of 9
 * element counts:
 *   { q_b, q_h, q_row,   kv_b, kv_h, kv_row,   o_b, o_h, o_row }
 * (K and V share one set).  Examples, for [B, N, H, d] tensors (token-major,
 * as most model code lays them out): q = {N*Hq*d, d, Hq*d}; for Q, K, V
 * sliced out of one packed projection [B, N, 3, H, d]: q = kv =
 * {N*3*H*d, d, 3*H*d} with k = q + H*d, v = q + 2*H*d.  lse stays dense
 * [B, Hq, N].  Every stride must be a non-negative multiple of 8 (16-byte
 * aligned rows), row strides at least d, and ((N + 127) * row + d) * 2 <
 * 2^31 (else ATTN_ERR_INVALID_ARG); distinct (b, h, i) must address distinct
 * rows of o (not checked).  Inputs may share memory with each other; the
 * outputs must not overlap the inputs or each other (checked on the extent
 * from base to last element).  Supported: ATTN_BF16 or ATTN_F16 (ATTN_F32 is
 * ATTN_ERR_UNSUPPORTED), d in {64, 128, 256}; every other convention is
 * attn_fwd's, and with the dense strides the result is attn_fwd's bit for
 * bit.
 */
attn_status attn_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                             const long long* strides, int B, int Hq, int Hkv, int N, int d,
                             int causal, float scale, attn_dtype dtype, void* stream);

/*
 * Backward on strided tensors, with the strides' meaning of attn_fwd_strided:
 * strides[0..2] address q and dq, strides[3..5] k, v, dk and dv,
 * strides[6..8] o and dout; lse and the workspace stay dense (the workspace
 * is attn_bwd_workspace_bytes(...) bytes).  Stride rules as for
 * attn_fwd_strided.  Inputs may share memory (one packed QKV buffer); dq, dk
 * and dv may be interleaved slices of one packed gradient buffer, so they are
 * only required to address disjoint elements (not checked), while each must
 * stay clear of every input and of the workspace (checked on extents).
 * Supported: ATTN_BF16 or ATTN_F16, d in {64, 128, 256}; with the dense
 * strides the result is attn_bwd's bit for bit.
 */
attn_status attn_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             void* workspace, const long long* strides, int B, int Hq, int Hkv,
                             int N, int d, int causal, float scale, attn_dtype dtype,
                             void* stream);

/*
 * Backward of attn_fwd_varlen: packed sequences as there (q, o, dout, dq
 * [Hq, T, d]; k, v, dk, dv [Hkv, T, d]; lse [Hq, T]; the same cu_seqlens,
 * nseq and max_seqlen), every sequence's gradients computed within that
 * sequence only.  workspace: attn_bwd_workspace_bytes(1, Hq, Hkv, T, d,
 * dtype) bytes (the row statistics of the T packed tokens), caller owned.
 * Offsets are clamped on the device as in attn_fwd_varlen.  Deterministic.
 * Supported: ATTN_BF16 or ATTN_F16, d in {64, 128, 256}, T <= 2^22,
 * nseq * Hq <= 2^24; nseq == 0, T == 0 or max_seqlen == 0 launches nothing.
 */
attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            void* workspace, const int* cu_seqlens, int nseq, int max_seqlen,
                            int Hq, int Hkv, int T, int d, int causal, float scale,
                            attn_dtype dtype, void* stream);

/*
 * attn_fwd_varlen / attn_bwd_varlen on packed-sequence tensors of any (head,
 * token) element strides, such as the token-major [T, H, d] layout or slices
 * of a packed [T, 3, H, d] QKV projection.
 *   strides[0..1]  (head, token) strides of q (and dq)
 *   strides[2..3]  (head, token) strides of k and v (and dk, dv)
 *   strides[4..5]  (head, token) strides of o (and dout)
 * lse stays dense [Hq, T]; the workspace is as for attn_bwd_varlen.  Every
 * stride must be a non-negative multiple of 8, token strides at least d, and
 * ((T + 127) * token_stride + d) * 2 < 2^31 (else ATTN_ERR_INVALID_ARG);
 * distinct (head, token) pairs must address distinct rows of every output
 * (not checked).  Inputs may share memory.  The forward's outputs must not
 * overlap the inputs or each other; the backward's gradients may be
 * interleaved slices of one packed buffer and are only checked against the
 * inputs, the workspace and cu_seqlens (on the extents from base to last
 * element).  Every other convention, including the supported types and head
 * dimensions, is that of the dense entry point, and with the dense [H, T, d]
 * strides (T*d, d for every tensor) the results are its results bit for bit.
 */
attn_status attn_fwd_varlen_strided(const void* q, const void* k, const void* v, void* o,
                                    float* lse, const int* cu_seqlens, const long long* strides,
                                    int nseq, int max_seqlen, int Hq, int Hkv, int T, int d,
                                    int causal, float scale, attn_dtype dtype, void* stream);
attn_status attn_bwd_varlen_strided(const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout, void* dq, void* dk,
                                    void* dv, void* workspace, const int* cu_seqlens,
                                    const long long* strides, int nseq, int max_seqlen, int Hq,
                                    int Hkv, int T, int d, int causal, float scale,
                                    attn_dtype dtype, void* stream);

/*
 * Measurement helper, not part of the attention path: the device's shader
 * clock while other work runs.  Launches nwg one-wave workgroups on
 * `stream`; workgroup i spins (sleeping) for `ticks` ticks of the 100 MHz
 * real-time counter and stores
 *   out[2i] = shader-clock cycles elapsed, out[2i+1] = real-time ticks elapsed,
 * so its mean clock over the spin is out[2i] / out[2i+1] * 100 MHz.
 * Workgroups are dealt round robin to the 8 XCDs, each with its own clock,
 * so nwg = 8 samples every XCD once.  Under sustained matrix-core load the
 * board lowers its clock to hold its power limit, and raises it again within
 * microseconds once the load stops, so the probe is meant for a second
 * stream beside the kernels being measured (bench.py does so).  out: device
 * pointer to 2*nwg unsigned 64-bit values, 8-byte aligned, written when the
 * kernel ends (asynchronously, like every launch here).  1 <= nwg <= 64 and
 * 1 <= ticks <= 200000000 (2 s); else ATTN_ERR_INVALID_ARG.
 */
attn_status attn_probe_clock(unsigned long long* out, int nwg, unsigned ticks, void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_str(attn_status s);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
