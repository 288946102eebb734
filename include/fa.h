/*
 * fa.h -- C ABI of the fused attention forward (and of the attention of new query
 * rows against a key/value cache) on AMD Instinct MI355X (gfx950).
 *
 * Computes, for every batch b, head h and query row i,
 *     O[b,h,i,:] = sum_j softmax_j(scale * Q[b,h,i,:] . K[b,h,j,:] + mask_ij) V[b,h,j,:]
 * tile by tile: a block of Q rows stays on chip while K/V column blocks stream
 * through LDS; a running row maximum and row sum (online softmax) rescale an
 * fp32 output accumulator, so the S x S score matrix never reaches memory.
 *
 * Defining passages:
 *   - the operation: Ascend C FlashAttention-2 tile-fusion page
 *     (ascendai.csdn.net), sections 1.1 and 1.2 (O_i = sum_j e^(P_ij - m_i) V_j
 *     / sum_j e^(P_ij - m_i), with m_i the row maximum); "FlashAttention on
 *     Ascend NPU: from principle to practice" (hwcomputing.csdn.net,
 *     6a0fe629), section "core idea: IO-aware" (scale 1/sqrt(head_dim) on QK^T);
 *   - the [B,H,S,D] fp16 tensors, causal flag and explicit scale:
 *     ops-transformer FlashAttention walkthrough (hwcomputing.csdn.net,
 *     6a0ef689), section on the complete operator (aclnn call example);
 *   - full / causal / (window_left, window_right) masks: catlass FlashAttention
 *     article (lnwmold.com/news/1200460), section "usage";
 *   - fp32 softmax and accumulation with fp16 inputs and output: the
 *     ops-transformer walkthrough, pitfall 3, and the tile-fusion page,
 *     section 10 (best practice).
 *
 * All functions are reentrant and thread-safe and allocate no memory
 * (fa_decode's workspace is the caller's). The only state is the per-device
 * address of the scratch array fa_decode_noalloc uses, looked up once.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Mask modes.
 *   FA_MASK_FULL   every key is visible (win_l, win_r ignored);
 *   FA_MASK_CAUSAL key j is visible from query i iff j <= i (win_l, win_r ignored);
 *   FA_MASK_WINDOW key j is visible iff i - win_l <= j <= i + win_r, both ends
 *                  inclusive; a negative win_l (win_r) leaves the left (right)
 *                  side unbounded, so (-1, 0) is causal and (-1, -1) is full. */
typedef enum {
    FA_MASK_FULL = 0,
    FA_MASK_CAUSAL = 1,
    FA_MASK_WINDOW = 2
} fa_mask_mode;

/* Element type of q, k, v and o. */
typedef enum {
    FA_DTYPE_FP16 = 0, /* IEEE binary16 */
    FA_DTYPE_BF16 = 1  /* bfloat16 */
} fa_dtype;

/* Pairings of the rotary embedding (fa_rope, fa_fwd_rope): dims (t, t + D/2)
 * or (2t, 2t + 1) form pair t, for t = 0 .. D/2 - 1. */
typedef enum {
    FA_ROPE_HALVES = 0,
    FA_ROPE_INTERLEAVED = 1
} fa_rope_mode;

/* Return codes. Every code except FA_ERR_HIP is returned before anything is
 * enqueued or written. */
typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum, non-finite
                                scale, output overlapping an input */
    FA_ERR_UNSUPPORTED = -2, /* head dimension other than 64 or 128 */
    FA_ERR_ALIGNMENT = -3,   /* q/k/v/o not 16-byte aligned, lse or an index array
                                not 4-byte aligned */
    FA_ERR_TOO_LARGE = -4,   /* a head's [S, D] block is 2^31 bytes or more, or the
                                launch grid or FLOP count would overflow */
    FA_ERR_HIP = -5          /* the HIP runtime rejected the kernel launch */
} fa_status;

/*
 * fa_fwd -- attention forward, O = softmax(scale * Q K^T + mask) V.
 *
 * q, k, v  device pointers, contiguous row-major [B, H, S, D] (D fastest), element
 *          type `dtype`; read only.
 * o        device pointer, [B, H, S, D] of `dtype`; fully overwritten. Each value
 *          is the fp32 result rounded to nearest even.
 * lse      device pointer to fp32 [B, H, S], or NULL to skip it; fully
 *          overwritten with the natural-log log-sum-exp of each row's visible
 *          scaled scores, log(sum_j exp(scale * q_i . k_j)).
 * B, H, S  batch, heads, sequence length (>= 0). If B*H*S == 0 the call does
 *          nothing and returns FA_OK without reading any pointer.
 * D        head dimension: 64 or 128.
 * scale    finite multiplier of Q K^T (1/sqrt(D) is the usual choice); any sign.
 * mask_mode, win_l, win_r  see fa_mask_mode.
 * dtype    fa_dtype of q, k, v and o.
 * stream   HIP stream on the current device; the call only enqueues work
 *          (asynchronous) and device faults surface at the caller's next
 *          synchronisation.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing,
 * needs no workspace and keeps no reference after return. o and lse must not
 * overlap q, k, v or each other (checked on the host).
 * Arithmetic: QK^T and PV run on fp16/bf16 matrix cores with fp32 accumulation;
 * softmax state is fp32. For PV the probabilities are rounded once to fp16
 * (fp16 inputs) or carried as two bf16 terms, the rounded value and the
 * rounded remainder, each multiplied by V (bf16 inputs: an 8-bit significand
 * alone is too coarse for the output bound when a few keys dominate a row).
 * The row sum (and so the LSE) adds the unrounded fp32 probabilities. Results
 * are bitwise deterministic for a given input, device and library build.
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int S, int D, float scale, int mask_mode, int win_l,
           int win_r, int dtype, hipStream_t stream);

/*
 * fa_visible_pairs -- number of (query, key) pairs of one S x S head that the
 * mask leaves visible (S >= 0). Returns the count, or a negative fa_status.
 */
int64_t fa_visible_pairs(int S, int mask_mode, int win_l, int win_r);

/*
 * fa_fwd_flops -- the algorithmic FLOPs of one fa_fwd call: 4 * D * B * H *
 * fa_visible_pairs(S, ...), counting a multiply-add as 2 FLOPs for each of the
 * two products QK^T and PV over visible pairs only. Returns the count, or a
 * negative fa_status.
 */
int64_t fa_fwd_flops(int B, int H, int S, int D, int mask_mode, int win_l, int win_r);

/*
 * fa_fwd_schedule -- the work plan fa_fwd uses for these arguments on a GPU
 * with n_cu compute units, without launching anything (host only; for tests
 * and tools). The query rows of each head are cut into work items (256 rows,
 * or 128 under the key-split layout of small grids); a persistent grid of
 * workgroups runs them from per-XCD lists in snake order (the tile-fusion
 * page's host-side grid and its causal block skipping, Ascend C
 * FlashAttention-2 page, sections 6 and 7, applied per item). Writes up to
 * max_items entries of 6 int32 each to `items` (host memory, caller-owned;
 * may be NULL when max_items is 0): workgroup, round, head b*H + h, first
 * query row, rows per item, key tiles the item walks. Returns the number of
 * entries (which may exceed max_items), or a negative fa_status for the
 * argument errors fa_fwd would report (pointer checks aside).
 */
int64_t fa_fwd_schedule(int B, int H, int S, int D, int mask_mode, int win_l, int win_r,
                        int n_cu, int32_t *items, int64_t max_items);

/*
 * fa_fwd_varlen -- fa_fwd over a batch of sequences of different lengths
 * packed token after token: sequence b holds tokens cu_seqlens[b] ..
 * cu_seqlens[b+1] - 1 of the packed tensors and attends only within itself,
 * its token cu_seqlens[b] + i being its query/key row i (the mask applies to
 * those row numbers). Defining passage: Ascend C FlashAttention-2 tile-fusion
 * page (ascendai.csdn.net), section 4.1 (data structures), which takes the
 * input as contiguous [total_tokens, H, D]; the per-sequence attention is
 * fa_fwd's.
 *
 * q, k, v      device pointers, contiguous [total_tokens, H, D] of `dtype`
 *              (D fastest, then heads, then tokens); read only.
 * o            device pointer, [total_tokens, H, D] of `dtype`; every token
 *              that lies in a sequence is overwritten (RNE), others are not
 *              touched.
 * lse          device pointer to fp32 [total_tokens, H], or NULL; written like o.
 * cu_seqlens   device pointer, int32 [nseq + 1], non-decreasing, cu_seqlens[0]
 *              normally 0 and cu_seqlens[nseq] <= total_tokens; read only. The
 *              kernel clamps each offset into [0, total_tokens] (and each end to
 *              at least its start) and attends over at most max_seqlen tokens of
 *              a sequence, so no bad value makes it touch memory outside the
 *              tensors; rows of overlapping sequences get unspecified values.
 * nseq         number of sequences (>= 0).
 * max_seqlen   host-side bound on every sequence's length (>= 0); tokens past it
 *              are not written. If nseq*H*max_seqlen == 0 or total_tokens == 0
 *              the call does nothing and returns FA_OK.
 * total_tokens rows of the packed tensors (>= 0).
 * H, D, scale, mask_mode, win_l, win_r, dtype, stream: as for fa_fwd.
 *
 * Limits: max_seqlen * H * D * 2 < 2^31 (FA_ERR_TOO_LARGE otherwise).
 * cu_seqlens needs 4-byte alignment and must not overlap o or lse.
 * Ownership and arithmetic as fa_fwd; each sequence's result is bitwise the
 * one fa_fwd gives for that sequence alone in [1, H, L, D] layout.
 */
int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int32_t *cu_seqlens, int nseq, int max_seqlen, int total_tokens,
                  int H, int D, float scale, int mask_mode, int win_l, int win_r,
                  int dtype, hipStream_t stream);

/*
 * fa_fwd_varlen_flops -- the algorithmic FLOPs of one fa_fwd_varlen call:
 * the sum over sequences of 4 * D * H * fa_visible_pairs(length). cu_seqlens is
 * a HOST pointer to int32 [nseq + 1] (non-negative, non-decreasing; otherwise
 * FA_ERR_INVALID_ARG). Returns the count, or a negative fa_status.
 */
int64_t fa_fwd_varlen_flops(const int32_t *cu_seqlens, int nseq, int H, int D,
                            int mask_mode, int win_l, int win_r);

/*
 * fa_bwd -- the attention backward pass: the gradients dQ, dK, dV of
 * O = softmax(scale * Q K^T + mask) V for a given dO = dL/dO, from the
 * forward's O and LSE (the state the forward keeps):
 *     P_ij = exp(scale q_i . k_j - LSE_i) on visible pairs, 0 elsewhere,
 *     D_i = dO_i . O_i,   dS_ij = P_ij (dO_i . v_j - D_i),
 *     dV_j = sum_i P_ij dO_i,  dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
 * Defining passage: ops-transformer FlashAttention walkthrough
 * (hwcomputing.csdn.net, 6a0ef689), closing remark (the backward needs the
 * forward's intermediate state), read as the gradient of fa_fwd's definition
 * recomputing P from the saved LSE.
 *
 * q, k, v, o, dout  device pointers, contiguous [B, H, S, D] of `dtype`, 16-byte
 *             aligned; o and lse as fa_fwd returned them for q, k, v and the same
 *             scale and mask; read only.
 * lse         device pointer to fp32 [B, H, S] (natural log); read only.
 * dq, dk, dv  device pointers, [B, H, S, D] of `dtype`, 16-byte aligned; fully
 *             overwritten (fp32 accumulation, rounded RNE once).
 * workspace   device memory of at least fa_bwd_workspace_bytes(B, H, S) bytes,
 *             4-byte aligned (it receives D_i); contents on entry do not matter.
 * B, H, S, D, scale, mask_mode, win_l, win_r, dtype, stream: as for fa_fwd.
 * Outputs and workspace must not overlap any input or each other (checked).
 * Arithmetic: S, dP, dV, dK, dQ on fp16/bf16 matrix cores with fp32
 * accumulation; P and dS are formed in fp32 and rounded to `dtype` as MFMA
 * operands. Deterministic: every output element is owned by one workgroup
 * (no atomics). Returns FA_OK or a negative fa_status.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, int B, int H, int S, int D,
           float scale, int mask_mode, int win_l, int win_r, int dtype, void *workspace,
           int64_t workspace_bytes, hipStream_t stream);

/* fa_bwd_workspace_bytes -- workspace fa_bwd needs: 4 * B * H * S bytes (or a
 * negative fa_status). */
int64_t fa_bwd_workspace_bytes(int B, int H, int S);

/* fa_bwd_flops -- algorithmic FLOPs of one fa_bwd call: the five products over
 * the visible pairs, 10 * D * B * H * fa_visible_pairs(S, ...) (2.5 times
 * fa_fwd_flops). Returns the count, or a negative fa_status. */
int64_t fa_bwd_flops(int B, int H, int S, int D, int mask_mode, int win_l, int win_r);

/*
 * fa_rope -- rotary position embedding (RoPE) of a [B, H, S, D] tensor: pair
 * t of row s of every head (see fa_rope_mode) turns by the angle whose cosine
 * and sine are cos_table[s * D/2 + t] and sin_table[s * D/2 + t]:
 *     y[a] = x[a] c - x[b] s,   y[b] = x[b] c + x[a] s,
 * computed in fp32 from the exact inputs and rounded once (RNE) to `dtype`.
 * Defining passage: Ascend C FlashAttention-2 tile-fusion page
 * (ascendai.csdn.net), section 9 (RoPE applied to Q and K from a cos/sin
 * table), read as the usual rotary embedding.
 *
 * x, y        device pointers, contiguous [B, H, S, D] of `dtype`, 16-byte
 *             aligned; y may be x (in place), otherwise they must not overlap.
 * cos_table, sin_table
 *             device pointers to fp32 [n_pos, D/2] (row = position), 16-byte
 *             aligned, n_pos >= S; read only; must not overlap y.
 * rope_mode   fa_rope_mode. B, H, S >= 0 (B*H*S == 0: nothing done); D 64 or
 *             128; dtype, stream as for fa_fwd.
 * Limits: B*H*S*D/16 < 2^31. Returns FA_OK or a negative fa_status.
 */
int fa_rope(const void *x, void *y, const float *cos_table, const float *sin_table,
            int n_pos, int rope_mode, int B, int H, int S, int D, int dtype,
            hipStream_t stream);

/*
 * fa_fwd_rope -- fa_fwd of the rotary-embedded q and k: row i of q and of k
 * turned as fa_rope does at position i, then the attention (v unrotated).
 * Defining passage: the tile-fusion page, section 9, which fuses the rotation
 * into the loads of the Q and K tiles. Here the rotation of each query row is
 * applied in registers as the row enters the kernel; k is rotated once, by
 * fa_rope, into k_rot (each key tile is streamed by several query tiles, so
 * rotating it on every load would repeat the work) and the attention reads
 * k_rot. The rotated keys are the ones a key/value cache stores.
 *
 * k_rot       device pointer, [B, H, S, D] of `dtype`, 16-byte aligned: receives
 *             the rotated k; may be k itself (rotated in place), otherwise must
 *             not overlap k; must not overlap q, v, o, lse or the tables.
 * cos_table, sin_table, n_pos, rope_mode  as for fa_rope (n_pos >= S).
 * Every other argument, and the arithmetic of the attention, as for fa_fwd;
 * the rotated query rows are rounded to `dtype` before QK^T, as the rotated
 * keys are. All checks run before anything is enqueued.
 */
int fa_fwd_rope(const void *q, const void *k, const void *v, void *o, float *lse,
                void *k_rot, const float *cos_table, const float *sin_table, int n_pos,
                int rope_mode, int B, int H, int S, int D, float scale, int mask_mode,
                int win_l, int win_r, int dtype, hipStream_t stream);

/*
 * fa_decode -- attention of Sq new query rows against a key/value cache
 * (incremental decoding): O = softmax(scale * Q K^T + mask) V, where query row i
 * sits at position Sk - Sq + i of its sequence and the cache holds positions
 * 0 .. Sk-1, the new rows' own keys included; the mask rules of fa_fwd apply at
 * that position (so FA_MASK_CAUSAL lets row i see keys 0 .. Sk - Sq + i).
 * Defining passage: "FlashAttention on Ascend NPU: from principle to practice"
 * (hwcomputing.csdn.net, 6a0fe629), section "optimisation 4: KV-cache reuse",
 * read as attention of each new row over every visible cached key.
 *
 * q        device pointer, contiguous [B, H, Sq, D] of `dtype`; read only.
 * k, v     device pointers, contiguous [B, H, Sk, D] of `dtype` (the cache); read only.
 * o        device pointer, [B, H, Sq, D] of `dtype`; fully overwritten (RNE).
 * lse      device pointer to fp32 [B, H, Sq] (natural log), or NULL.
 * B, H     >= 0. Sq: 0 .. 32 query rows, Sq <= Sk. If B*H*Sq == 0 the call does
 *          nothing and returns FA_OK. D: 64 or 128. scale, mask_mode, win_l,
 *          win_r, dtype, stream: as for fa_fwd.
 * workspace, workspace_bytes
 *          device memory for per-split partial results, at least
 *          fa_decode_workspace_bytes(...) bytes and 16-byte aligned; may be NULL
 *          when that size is 0. Owned by the caller; the call only uses it
 *          until the enqueued work completes; its contents on entry do not
 *          matter and on exit are unspecified.
 *
 * The visible cache range of each head is cut into splits processed by
 * separate workgroups; each writes its normalised partial output and LSE to
 * the workspace and a second kernel merges the splits of each row,
 * LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s. The number of
 * splits depends on the shape and the current device's CU count, so call
 * fa_decode_workspace_bytes with the same device current. Same arithmetic,
 * determinism, ownership and error rules as fa_fwd; additionally
 * FA_ERR_UNSUPPORTED for Sq > 32, FA_ERR_INVALID_ARG for Sq > Sk, a missing or
 * short workspace, or o, lse or the workspace overlapping an input or each
 * other. Returns FA_OK or a negative fa_status.
 */
int fa_decode(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int Sq, int Sk, int D, float scale, int mask_mode, int win_l,
              int win_r, int dtype, void *workspace, int64_t workspace_bytes,
              hipStream_t stream);

/*
 * fa_decode_workspace_bytes -- bytes of workspace fa_decode needs for these
 * arguments on the current device (0 when one split suffices and none is
 * needed). Returns the size, or the negative fa_status fa_decode would return
 * for these arguments.
 */
int64_t fa_decode_workspace_bytes(int B, int H, int Sq, int Sk, int D, int mask_mode, int win_l,
                                  int win_r);

/*
 * fa_decode_noalloc -- fa_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The split partials go to a scratch
 * array the library holds in device memory, one copy per GPU, alive until the
 * process ends; the call itself allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). The first call on a device looks up that
 * device's copy (hipGetSymbolAddress); later calls reuse the address.
 *
 * Arguments, layout, ownership, results and error rules: as fa_decode with
 * the workspace taken from the scratch array. Additionally FA_ERR_TOO_LARGE
 * when the split partials would exceed the scratch array's 24 MiB
 * (fa_decode_workspace_bytes(...) > 25165824; no shape does on a 256-CU
 * device), and FA_ERR_HIP when the array's address cannot be looked up.
 * Nothing in the array needs to start at zero: every partial the merge
 * reads is written by the same call. Calls on one GPU share its array, so
 * calls that may overlap in time on one GPU (other streams, other threads)
 * race and give undefined results; calls on one stream are ordered and safe.
 */
int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int H, int Sq, int Sk, int D, float scale, int mask_mode,
                      int win_l, int win_r, int dtype, hipStream_t stream);

/*
 * fa_decode_paged -- fa_decode over a paged key/value cache (serving layout).
 * The cached keys and values of all sequences live in page pools
 * k_pages, v_pages: [num_pages, page_size, H, D] of `dtype`; key j of sequence b
 * is row j % page_size of page block_table[b * max_pages + j / page_size], and
 * sequence b caches seq_lens[b] keys (its new rows are its last Sq positions).
 * Defining passage: as fa_decode; the paged layout is the serving form of the
 * same cache ("optimisation 4: KV-cache reuse" keeps the cache across steps).
 *
 * block_table  device pointer, int32 [B, max_pages]; read only. Entries past a
 *              sequence's pages are not read. An entry outside [0, num_pages)
 *              makes that page's keys read as zero (nothing outside the pools
 *              is touched).
 * seq_lens     device pointer, int32 [B]; read only; each value is clamped to
 *              [0, max_seq_len]. A row at a negative position (seq_lens[b] < Sq)
 *              sees no key: its output is 0 and its LSE -inf.
 * max_seq_len  host-side bound on seq_lens (sizes the split); Sq <= max_seq_len
 *              <= max_pages * page_size.
 * num_pages    pages in each pool (>= 1); page_size a positive multiple of 32.
 * Other arguments, the workspace (size from fa_decode_paged_workspace_bytes) and
 * the error rules as fa_decode; FA_ERR_UNSUPPORTED for a page_size that is not a
 * positive multiple of 32, FA_ERR_ALIGNMENT for block_table or seq_lens not
 * 4-byte aligned.
 */
int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages, void *o, float *lse,
                    const int32_t *block_table, const int32_t *seq_lens, int B, int H, int Sq,
                    int max_seq_len, int D, int num_pages, int page_size, int max_pages,
                    float scale, int mask_mode, int win_l, int win_r, int dtype,
                    void *workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * fa_decode_paged_workspace_bytes -- workspace fa_decode_paged needs on the
 * current device for these arguments (0 if none), or a negative fa_status.
 */
int64_t fa_decode_paged_workspace_bytes(int B, int H, int Sq, int max_seq_len, int D,
                                        int mask_mode, int win_l, int win_r);

/*
 * fa_decode_rope, fa_decode_paged_rope -- fa_decode and fa_decode_paged with
 * the rotary embedding of the new query rows: row i (at position
 * Sk - Sq + i, or seq_lens[b] - Sq + i for a paged sequence) turns as fa_rope
 * turns row position, in fp32, and enters Q K^T rounded to `dtype`. The cache
 * holds keys already rotated (as fa_fwd_rope's k_rot or fa_rope leave them),
 * so they are read as given. Defining passage: the tile-fusion page, section 9
 * (RoPE applied as the Q and K tiles load; keys are rotated once, when cached).
 *
 * cos_table, sin_table, n_pos, rope_mode  as for fa_rope, with n_pos >= Sk (or
 * max_seq_len): positions past the tables' end never occur; a row at a
 * negative position (a paged sequence shorter than Sq) uses row 0 and sees no
 * key anyway. The tables must not overlap o, lse or the workspace.
 * Every other argument, the workspace (same size as without RoPE) and the
 * error rules as fa_decode / fa_decode_paged.
 */
int fa_decode_rope(const void *q, const void *k, const void *v, void *o, float *lse,
                   const float *cos_table, const float *sin_table, int n_pos, int rope_mode,
                   int B, int H, int Sq, int Sk, int D, float scale, int mask_mode, int win_l,
                   int win_r, int dtype, void *workspace, int64_t workspace_bytes,
                   hipStream_t stream);
int fa_decode_paged_rope(const void *q, const void *k_pages, const void *v_pages, void *o,
                         float *lse, const int32_t *block_table, const int32_t *seq_lens,
                         const float *cos_table, const float *sin_table, int n_pos,
                         int rope_mode, int B, int H, int Sq, int max_seq_len, int D,
                         int num_pages, int page_size, int max_pages, float scale,
                         int mask_mode, int win_l, int win_r, int dtype, void *workspace,
                         int64_t workspace_bytes, hipStream_t stream);

/*
 * fa_decode_flops -- algorithmic FLOPs of one fa_decode call: 4 * D * B * H *
 * (visible (row, key) pairs), rows at positions Sk - Sq .. Sk - 1. Returns the
 * count, or a negative fa_status.
 */
int64_t fa_decode_flops(int B, int H, int Sq, int Sk, int D, int mask_mode, int win_l, int win_r);

/* fa_strerror -- static description of a status code (never NULL). */
const char *fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
