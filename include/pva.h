/*
 * pva.h — packed variable-length mixed-mask attention on MI355X (gfx950).
 *
 * The operation (forward only, inference):
 *   Several sequences are packed back to back along one token axis, without
 *   padding, and addressed by prefix sums of their lengths ("cu_seqlens").
 *   This replaces the padded batch plus explicit (bsz, 1, seqlen, seqlen)
 *   boolean mask described in "[RFC]: HunyuanImage 3.0 deployment",
 *   Motivation (1), by the packed cu_seqlens layout of that RFC's Proposed
 *   Change P0 ("Packed Attention for Multi-Request Batching").
 *
 *   Sequence s holds T_s text tokens followed by I_s image tokens,
 *   L_s = T_s + I_s. Its mask is the RFC's Generalized Causal Attention
 *   (Proposed Change P0, attention mask challenge; Model structure, item 1):
 *   text row i (i < T_s) attends to keys 0..i; image rows attend to all L_s
 *   keys of their sequence (the whole text prefix and every image token).
 *   No row attends across sequences. For every sequence s and head h:
 *       O = softmax(scale * Q K^T + mask) V,
 *   accumulated in fp32, rows with no allowed key defined as zero (no such
 *   row exists for L_s >= 1 under this mask).
 *
 * Layout: Q, K, V and O are [N, H, D] row-major (D contiguous), N = sum L_s,
 * in pack order. All heads share one sequence structure (no GQA).
 *
 * Generalization (pva_seg_desc_build_segments): a sequence may be any list of
 * text (causal) and image (full) segments, and only a suffix of it may be
 * queried, with Q and O holding just the queried rows. With
 * pva_seg_desc_build_kv_chunk, K and V may hold just a chunk of each
 * sequence's keys; packed_attn_fwd_partial (bf16) or
 * packed_attn_fwd_partial_fp8 then also returns the rows' log-sum-exp and
 * pva_merge_partials combines the chunks' results, or
 * packed_attn_fwd_partial_accumulate(_fp8) folds each chunk into a running
 * result as it is computed. packed_attn_fwd_paged reads K and V from a block
 * pool through a block table.
 *
 * Ownership: the caller owns every tensor and every stream. The library owns
 * only a pva_seg_desc (host copy + device work list), freed by
 * pva_seg_desc_free. No call allocates device memory except the descriptor
 * builders that upload a work list (pva_seg_desc_build, _build_segments,
 * _build_kv_chunk); pva_seg_desc_build_noalloc uses a fixed buffer instead.
 *
 * Errors: every entry point returns a pva_status (0 on success). Arguments
 * are validated on the host before any launch; nothing throws or aborts
 * across this boundary. pva_last_error() returns a thread-local message
 * for the last failing call on the calling thread. Kernel launches are
 * asynchronous: faults surface at the caller's next synchronisation.
 */
#ifndef PVA_H_
#define PVA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PVA_OK = 0,
  PVA_ERR_INVALID_ARG = -1, /* a size, pointer, alignment or value is out of range   */
  PVA_ERR_UNSUPPORTED = -2, /* a valid request the library does not implement (e.g. D) */
  PVA_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed              */
  PVA_ERR_NO_MEMORY = -4    /* host or device allocation failed                        */
} pva_status;

typedef enum { PVA_BF16 = 0, PVA_FP8_E4M3 = 1 } pva_dtype;

/* Segment kinds of the multi-segment Generalized Causal mask ("[RFC]:
 * HunyuanImage 3.0 deployment", Model structure item 1, which interleaves
 * text and image segments in one context): a token of a CAUSAL (text)
 * segment at position i sees keys 0..i of its sequence; a token of a FULL
 * (image) block [a, b) sees keys 0..b-1 (every earlier segment and its whole
 * block). */
typedef enum { PVA_SEG_CAUSAL = 0, PVA_SEG_FULL = 1 } pva_seg_kind;

/* Opaque, library-owned descriptor of one batch composition. */
typedef struct pva_seg_desc pva_seg_desc;

/*
 * Segment-descriptor builder (host). From per-sequence (text_len, image_len)
 * it derives cu_seqlens and, per query tile of BM rows and key tiles of BN
 * keys, the tile classes of the mask above: key tiles below k_full_end are
 * FULL (no masking), tiles from k_end on are SKIP (never visited), tiles in
 * between are PARTIAL (masked element-wise). This is the block-sparse form of
 * the mixed mask named in the RFC's attention mask challenge (Proposed Change
 * P0). It then orders the (sequence, head, query-tile) work items for the
 * varlen tile scheduler and uploads the work list to device memory with an
 * asynchronous copy on `stream` (a hipStream_t; NULL = the null stream).
 *
 *   text_len, image_len : host int32 [nseq], copied; T >= 0, I >= 0, T+I >= 1
 *   nseq                : >= 1, sum of lengths must fit in int32
 *   num_heads           : H >= 1, H * head_dim * N must fit in int64
 *   head_dim            : D in {64, 128} for PVA_BF16, 128 for PVA_FP8_E4M3
 *                         (every sequence needs L * H * D * e < 2^31, e = 2
 *                         bytes per bf16 element, 1 per fp8 code: one head's
 *                         rows are addressed with 32-bit byte offsets;
 *                         PVA_ERR_UNSUPPORTED otherwise)
 *   dtype               : element type of Q/K/V the descriptor will serve
 *   out                 : receives the descriptor on PVA_OK, NULL otherwise
 * The host arrays are not referenced after return. The descriptor must
 * outlive every launch that uses it (free only after those launches have
 * completed on their streams).
 */
int pva_seg_desc_build(const int32_t* text_len, const int32_t* image_len, int32_t nseq,
                       int32_t num_heads, int32_t head_dim, pva_dtype dtype, void* stream,
                       pva_seg_desc** out);

/*
 * Allocation-free variant of pva_seg_desc_build, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, planning and result, but
 * the descriptor's device work list and per-row key limits are copied into
 * a fixed buffer the library holds on each device
 * (PVA_NOALLOC_SCRATCH_BYTES bytes, kept until the process ends) instead
 * of a hipMalloc'ed one: no device memory is allocated or freed by this call
 * or by pva_seg_desc_free of its result (the host-side descriptor itself is
 * ordinary host memory).
 *   Size limit: round_up(32 * work items, 256) + 4 * packed tokens must not
 *   exceed PVA_NOALLOC_SCRATCH_BYTES (the mixed-resolution batch of 8
 *   sequences and 25,072 tokens at 32 heads needs 305 KB); a larger batch
 *   gets PVA_ERR_INVALID_ARG before anything is copied.
 *   One buffer per device: each call replaces the work list of the previous
 *   no-alloc descriptor of the current device (also when its upload then
 *   fails). Forward calls with that older descriptor are refused on the host
 *   with PVA_ERR_INVALID_ARG (rebuild it); descriptors from
 *   pva_seg_desc_build are not affected.
 *   Calls that overlap on one device race: a build that runs while a launch
 *   with the previous no-alloc descriptor of that device still executes on
 *   another stream changes the work list under it. Order them on one stream
 *   (the copy is issued on `stream`), or synchronise in between. A HIP graph
 *   that captured launches with a no-alloc descriptor reads the buffer when
 *   it is replayed (the host-side check does not run then): replay it only
 *   while that descriptor is still its device's current no-alloc one.
 * The upload is synchronised on `stream` before return, as in
 * pva_seg_desc_build.
 */
#define PVA_NOALLOC_SCRATCH_BYTES (4u << 20)
int pva_seg_desc_build_noalloc(const int32_t* text_len, const int32_t* image_len, int32_t nseq,
                               int32_t num_heads, int32_t head_dim, pva_dtype dtype, void* stream,
                               pva_seg_desc** out);

/* Same planning without touching any device: the result can be inspected
 * (accessors below) but not launched. For host-side tests and tools. */
int pva_seg_desc_build_host(const int32_t* text_len, const int32_t* image_len, int32_t nseq,
                            int32_t num_heads, int32_t head_dim, pva_dtype dtype,
                            pva_seg_desc** out);

/*
 * General builder: any number of segments per sequence (the multi-segment
 * Generalized Causal mask above), and optionally only a suffix of each
 * sequence queried. Queries then cover rows [q_start_s, L_s) of sequence s:
 * K and V still hold all L_s rows (a prefix computed once and reused, the
 * RFC's single "Prefix KV", Model structure item 1), while Q and O hold only
 * the queried rows, packed in sequence order (cu_seqlens_q below).
 *
 *   seg_len, seg_kind : host int32, all sequences' segments back to back
 *                       (sum of seg_count entries); lengths >= 0, kinds
 *                       PVA_SEG_CAUSAL or PVA_SEG_FULL; every sequence needs
 *                       at least one token
 *   seg_count         : host int32 [nseq], segments per sequence (>= 1)
 *   q_start           : host int32 [nseq] in [0, L_s], or NULL for all zero
 *   others            : as pva_seg_desc_build
 * (text_len, image_len) of pva_seg_desc_build is the case of two segments
 * {CAUSAL T_s, FULL I_s} with q_start = 0. A descriptor with any q_start > 0
 * is launched with packed_attn_fwd_varlen / _varlen_fp8 only.
 */
int pva_seg_desc_build_segments(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                                const int32_t* q_start, int32_t nseq, int32_t num_heads, int32_t head_dim,
                                pva_dtype dtype, void* stream, pva_seg_desc** out);

/*
 * Key-chunk builder: as pva_seg_desc_build_segments, but k and v hold only
 * the key rows [k_lo_s, k_hi_s) of each sequence (one rank's share of the
 * keys in Ring attention, "[RFC]: HunyuanImage 3.0 deployment", Proposed
 * Change P2; the Parallelism guide's Ring-Attention). cu_seqlens then
 * counts those chunk rows. A queried row attends to the allowed keys of its
 * mask row that fall in the chunk; a row with none gets O = 0 and
 * lse = -inf from packed_attn_fwd_partial.
 *   k_lo, k_hi : host int32 [nseq], 0 <= k_lo <= k_hi <= L_s
 * Launched with packed_attn_fwd_partial (or the varlen entry points).
 */
int pva_seg_desc_build_kv_chunk(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                                const int32_t* q_start, const int32_t* k_lo, const int32_t* k_hi, int32_t nseq,
                                int32_t num_heads, int32_t head_dim, pva_dtype dtype, void* stream,
                                pva_seg_desc** out);

/* Host-only planning of the key-chunk builder. */
int pva_seg_desc_build_kv_chunk_host(const int32_t* seg_len, const int32_t* seg_kind, const int32_t* seg_count,
                                     const int32_t* q_start, const int32_t* k_lo, const int32_t* k_hi,
                                     int32_t nseq, int32_t num_heads, int32_t head_dim, pva_dtype dtype,
                                     pva_seg_desc** out);

/* Host-only planning of the general builder (inspection, no device). */
int pva_seg_desc_build_segments_host(const int32_t* seg_len, const int32_t* seg_kind,
                                     const int32_t* seg_count, const int32_t* q_start, int32_t nseq,
                                     int32_t num_heads, int32_t head_dim, pva_dtype dtype,
                                     pva_seg_desc** out);

/* Host view of the descriptor's cu_seqlens (int32 [nseq + 1], offsets of the
 * sequences' K/V rows); valid until the descriptor is freed. */
int pva_seg_desc_cu_seqlens(const pva_seg_desc* desc, const int32_t** host_cu, int32_t* len);

/* Host view of the query-row offsets (int32 [nseq + 1]): cu_seqlens_q[s]
 * is the first Q/O row of sequence s. Equal to cu_seqlens when every
 * q_start is 0. Valid until freed. */
int pva_seg_desc_cu_seqlens_q(const pva_seg_desc* desc, const int32_t** host_cu_q, int32_t* len);

/* Host view of the key limits of the queried rows (int32 [total_q], in Q/O
 * row order): queried row r of sequence s may attend to the K/V rows
 * [0, lim) of that sequence held by k and v, lim = key_limits[r]
 * (row q_start_s + r - cu_seqlens_q[s] of the sequence). Non-decreasing within
 * a sequence. Valid until freed. */
int pva_seg_desc_key_limits(const pva_seg_desc* desc, const int32_t** key_limits, int32_t* len);

/* Useful multiply-add FLOPs over allowed (query, key) pairs of the queried
 * rows only: 4 * D * H * sum over queried rows of lim; for two segments and
 * q_start = 0 that is 4 * D * H * sum_s [T_s (T_s + 1) / 2 + I_s * L_s].
 * Returns -1 on NULL. */
int64_t pva_seg_desc_useful_flops(const pva_seg_desc* desc);

/* Tile shape the descriptor was planned with (query rows BM, keys BN). */
int pva_seg_desc_tile(const pva_seg_desc* desc, int32_t* block_m, int32_t* block_n);

/* Host view of the work list in launch order: int32 [n_items][8] records
 * {seq, head, q0, q_rows, k_full_end, k_end, qo_row, L}: query rows
 * [q0, q0 + q_rows) of sequence seq (row numbers within the sequence), key
 * tiles below k_full_end need no mask, tiles from k_end on are skipped,
 * qo_row is the Q/O row holding query row q0, L the K/V rows k and v hold
 * for the sequence (its length; the chunk's rows for a key-chunk descriptor);
 * seq = -1 marks an empty slot that keeps the XCD alignment of the list.
 * Valid until freed. */
int pva_seg_desc_work_items(const pva_seg_desc* desc, const int32_t** items, int32_t* n_items);

/* Free a descriptor (NULL is a no-op). Releases its device work list with
 * hipFree, which synchronises the device. */
void pva_seg_desc_free(pva_seg_desc* desc);

/*
 * Packed mixed-mask attention forward, bf16 in, fp32 accumulate, bf16 out.
 *
 *   q, k, v    : device bf16 [N, H, D], 16-byte aligned
 *   cu_seqlens : device int32 [nseq + 1] equal to the descriptor's
 *   seg_desc   : built by pva_seg_desc_build with dtype PVA_BF16
 *   scale      : softmax scale (finite, > 0), usually 1/sqrt(D); the scaled
 *                scores scale * q.k must stay finite in fp32
 *   out        : device bf16 [N, H, D], 16-byte aligned; every row of every
 *                sequence is written; nothing outside [N, H, D] is touched
 *   stream     : hipStream_t to launch on (NULL = null stream), a stream of
 *                the current device
 * The descriptor may come from either builder as long as every q_start is 0
 * (else PVA_ERR_INVALID_ARG: use packed_attn_fwd_varlen). Every forward
 * entry point requires the current device to be the one the descriptor was
 * built on (its work list lives there); else PVA_ERR_INVALID_ARG.
 * Asynchronous; allocates nothing. With the environment variable PVA_CHECK=1
 * the device cu_seqlens is copied back (synchronously) and compared with the
 * descriptor's before the launch.
 */
int packed_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                    const pva_seg_desc* seg_desc, float scale, void* out, void* stream);

/*
 * FP8 variant: q, k, v are OCP E4M3FN codes [N, H, D] (16-byte aligned) with
 * one fp32 dequantisation scale per (sequence, head) and tensor
 * (q_scale/k_scale/v_scale: device float [nseq * H], index s * H + h), so
 * that the value of a code x is decode(x) * scale. Scales are finite and
 * >= 0 (they are read on the device, not checked); a zero q or k scale
 * makes every allowed score of that slice equal, a zero v scale its output
 * zero. The fp8 MFMA sums each 64-term block of a dot product with limited
 * precision (terms far below the block's largest product lose low bits), so
 * scores carry errors of about 2^-13 of their largest product: harmless at
 * the usual 1/sqrt(D), a tenth of a log2 unit between nearly tied keys at
 * softmax scales around 100. QK^T and PV run on fp8
 * MFMA; the probabilities are quantised to E4M3 for PV; out is bf16
 * [N, H, D]. Otherwise as packed_attn_fwd; the descriptor must have been
 * built with dtype PVA_FP8_E4M3.
 */
int packed_attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                        const float* k_scale, const float* v_scale, const int32_t* cu_seqlens,
                        const pva_seg_desc* seg_desc, float scale, void* out, void* stream);

/*
 * Forward over a descriptor from pva_seg_desc_build_segments (or any other):
 * q and out hold the queried rows only ([cu_seqlens_q[nseq], H, D]), k and v
 * whole sequences ([cu_seqlens[nseq], H, D]). cu_seqlens_q / cu_seqlens_k
 * are device int32 [nseq + 1] equal to the descriptor's (checked with
 * PVA_CHECK=1). Every queried row is written; nothing else in out is
 * touched. Otherwise as packed_attn_fwd.
 * Tensors of zero rows may be passed as NULL, in this and every other
 * forward call: q and out (with out_f32, lse, o_acc and lse_acc) when the
 * descriptor queries no row (every q_start = L: the call checks its
 * arguments and launches nothing), k and v when its key chunks hold no rows.
 */
int packed_attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale, void* out,
                           void* stream);

/* FP8 variant of packed_attn_fwd_varlen (scales as in packed_attn_fwd_fp8). */
int packed_attn_fwd_varlen_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                               const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                               void* out, void* stream);

/*
 * Partial forward for Ring-style combination (bf16 descriptors): writes O in
 * fp32 (out_f32: device float [total_q, H, D], 16-byte aligned) and the
 * log-sum-exp of every queried row's scaled scores over the keys it sees
 * (lse: device float [total_q, H], index row * H + h, 4-byte aligned):
 * lse = log(sum_j exp(scale * q.k_j)), -inf (and O = 0) for a row with no
 * allowed key among the K/V rows held. Otherwise as packed_attn_fwd_varlen.
 */
int packed_attn_fwd_partial(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                            float* out_f32, float* lse, void* stream);

/*
 * FP8 variant of packed_attn_fwd_partial (scales as in packed_attn_fwd_fp8;
 * the descriptor must have been built with dtype PVA_FP8_E4M3). The dot
 * products are those of the dequantised inputs, q.k_j = q_s k_s (codes'
 * product), and O and lse use the weights PV applied, i.e. the E4M3
 * probabilities, so the chunks of one row merge exactly as in the bf16 case.
 */
int packed_attn_fwd_partial_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                                float* out_f32, float* lse, void* stream);

/*
 * Partial forward over one key chunk that folds the chunk into a running
 * result, the online form of the combining step of Ring attention
 * ("[RFC]: HunyuanImage 3.0 deployment", Proposed Change P2): per queried
 * row, with (O_c, lse_c) this chunk's partial result as packed_attn_fwd_partial
 * would write it and (O_acc, lse_acc) the running one,
 *   lse = log(exp(lse_acc) + exp(lse_c)),
 *   O   = exp(lse_acc - lse) O_acc + exp(lse_c - lse) O_c.
 *   o_acc   : device float [total_q, H, D], 16-byte aligned: the running O
 *             (from packed_attn_fwd_partial or an earlier call of this one)
 *   lse_acc : device float [total_q, H], 4-byte aligned, disjoint from
 *             o_acc: its log-sum-exp; -inf marks a row no chunk has given a
 *             key yet, whose o_acc row then does not enter the result (it
 *             may hold anything, NaN included)
 *   out     : NULL: the merged O goes back to o_acc; else device bf16
 *             [total_q, H, D], 16-byte aligned, disjoint from o_acc and
 *             lse_acc: the merged O goes there in bf16 (the last chunk) and
 *             o_acc is left as it was
 * lse_acc receives the merged log-sum-exp in both cases. Overlapping
 * buffers are refused (PVA_ERR_INVALID_ARG) before anything is launched.
 * Starting from lse_acc = -inf everywhere, one call per chunk gives the
 * result of packed_attn_fwd_partial + pva_merge_partials without the
 * per-chunk fp32 outputs and the merge pass. Calls on one o_acc must be
 * ordered (one stream). Other arguments and errors as
 * packed_attn_fwd_partial.
 */
int packed_attn_fwd_partial_accumulate(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                                       float* o_acc, float* lse_acc, void* out, void* stream);

/* FP8 variant of packed_attn_fwd_partial_accumulate (inputs and scales as in
 * packed_attn_fwd_partial_fp8). */
int packed_attn_fwd_partial_accumulate_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                                           const float* k_scale, const float* v_scale, const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, const pva_seg_desc* seg_desc, float scale,
                                           float* o_acc, float* lse_acc, void* out, void* stream);

/*
 * Forward with K and V in a paged pool (the scheduler-managed paged KV mode
 * of "HunyuanImage-3.0-Instruct DiT Image Generation on 4x GPU", section
 * "Scheduler-managed paged KV": unquantised bf16 K/V in a fixed physical
 * pool, one logical row per CFG branch):
 *   k_pool, v_pool : device bf16 [num_blocks, block_size, H, D], 16-byte aligned
 *   block_table    : device int32 [nseq * table_stride]; key rows
 *                    [b * block_size, (b + 1) * block_size) of sequence s live
 *                    in pool block block_table[s * table_stride + b]
 *   table_stride   : >= ceil(L_s / block_size) for every sequence
 *   block_size     : a power of two, >= 32 (the key tile) and <= 2^20
 *   num_blocks     : blocks in each pool (>= 1); entries outside [0, num_blocks)
 *                    are clamped into the pool by the kernel (garbage in,
 *                    garbage out, but no access outside the pool); with
 *                    PVA_CHECK=1 the table is checked on the host first
 *   q, out, cu_seqlens_q, seg_desc : as packed_attn_fwd_varlen (bf16, whole
 *                    sequences: a descriptor from pva_seg_desc_build or
 *                    pva_seg_desc_build_segments, any q_start)
 * Pool rows past a sequence's end are never read into the result (they are
 * zero-filled in the kernel), so partly used blocks need no clearing.
 */
int packed_attn_fwd_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                          int32_t table_stride, int32_t block_size, int32_t num_blocks,
                          const int32_t* cu_seqlens_q, const pva_seg_desc* seg_desc, float scale, void* out,
                          void* stream);

/*
 * Merge of n_parts partial results over disjoint key sets (the combining
 * step of Ring attention, Proposed Change P2): for each of `rows`
 * (query, head) rows,
 *   lse = log sum_c exp(lse_c),   O = sum_c exp(lse_c - lse) O_c;
 * rows whose parts are all -inf give O = 0 and lse = -inf.
 *   o_parts   : device float [n_parts, rows, head_dim], 16-byte aligned
 *               (part c's O from packed_attn_fwd_partial is one [rows, D] slab)
 *   lse_parts : device float [n_parts, rows], 4-byte aligned
 *   n_parts   : >= 1; rows >= 0 (with rows = 0 the pointers may be NULL);
 *               head_dim in {64, 128}
 *   out       : device bf16 [rows, head_dim], 16-byte aligned
 *   lse_out   : device float [rows], or NULL
 * Asynchronous on `stream`; allocates nothing.
 */
int pva_merge_partials(const float* o_parts, const float* lse_parts, int32_t n_parts, int64_t rows,
                       int32_t head_dim, void* out, float* lse_out, void* stream);

/*
 * Workgroup timeline, for performance analysis (timing build only).
 * libpva_timeline.so is this library compiled with PVA_WG_TIMELINE: the same
 * calls and kernels, except that each launch of a forward kernel also writes
 * one record per work item (workgroup) into a fixed per-device buffer of that
 * kernel, PVA_TIMELINE_FIELDS uint64 per record, at the item's index in the
 * work list:
 *   [0] real-time counter (100 MHz) when the workgroup starts
 *   [1] the same after its prologue (work item, key limits, Q and the first
 *       K/V tiles in place)
 *   [2] the same after its tile loop (the first wave's last key tile)
 *   [3] the same at its end (output stored)
 *   [4] [5] shader-clock counter after the prologue and after the loop
 *   [6] HW_ID of the wave (CU in bits 11:8, shader array bit 12, engine
 *       bits 15:13), [7] XCC_ID (XCD in bits 3:0)
 *   [8] key tiles the first wave computes, [9] key tiles of the item
 *   [10] workgroup index, [11] 1 once written (empty work-list slots write
 *       nothing)
 *   kernel : PVA_BF16 (the contiguous and the paged bf16 kernels share one
 *            buffer) or PVA_FP8_E4M3
 * pva_timeline_clear zeroes the kernel's records on the current device;
 * pva_timeline_read copies records [0, n_records) to host memory
 * (n_records <= PVA_TIMELINE_MAX_ITEMS). Both synchronise the device. A
 * launch overwrites the records of its own work items only, so clear before
 * the launch to be read. The library's own build returns
 * PVA_ERR_UNSUPPORTED from both.
 */
#define PVA_TIMELINE_FIELDS 12
#define PVA_TIMELINE_MAX_ITEMS 131072
int pva_timeline_clear(pva_dtype kernel);
int pva_timeline_read(pva_dtype kernel, uint64_t* host_records, int64_t n_records);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* pva_last_error(void);

/* Library version string. */
const char* pva_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PVA_H_ */
