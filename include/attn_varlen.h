/*
 * attn_varlen.h: C ABI of the MI355X (gfx950) packed variable-length
 * attention library (libattn_varlen.so): the forward, and its backward
 * (section "Backward" below).
 *
 * Operation. For every segment b, with query rows [cu_q[b], cu_q[b+1]) and
 * key/value rows [cu_k[b], cu_k[b+1]), every head h and every query row i of
 * the segment:
 *     O[i,h,:] = softmax_j(scale * Q[i,h,:] . K[j,h,:]) V[j,h,:]   (j in segment b)
 *     LSE[h,i] = ln sum_j exp(scale * Q[i,h,:] . K[j,h,:])
 * This is the varlen flash-attention forward with its (out, lse) return as
 * used on the "[FA4] cute varlen backward: int32 overflow in _bwd_preprocess
 * ..." page ("Real-world trigger", repro script forward call) and the
 * "[FA4][SM120] flash_attn_varlen_func ... illegal memory access at >=4 varlen
 * segments" page ("Bug 2 details": packed q [35280,56,128], cu_seqlens_q,
 * max_seqlen_q/k). Equal head counts for Q and K/V; non-causal unless the
 * ATTN_VARLEN_CAUSAL option (below) is given.
 *
 * Layout. q, out: [total_q, H, D]; k, v: [total_k, H, D]; bf16; the D
 * dimension is contiguous (stride 1); the token-row and head strides are free
 * (in ELEMENTS, int64), e.g. the [N,H,D] views with row stride 9728 of the
 * _bwd_preprocess page. lse: fp32, element (h, i) at lse[h*lse_head + i].
 * Every offset is formed in 64-bit arithmetic, so element offsets past 2^31
 * and byte offsets past 2^32 are fine (that page's "Verified sample":
 * 225304 * 9728 = 2,191,757,312 must not wrap).
 *
 * Ownership. The caller owns every buffer and the stream. The library keeps
 * no pointer after a call returns, allocates no device memory and launches
 * work only on the given stream (asynchronously). out/lse must not overlap
 * q/k/v element-wise.
 *
 * Errors. Every entry point returns 0 on success or a negative
 * ATTN_VARLEN_E* code; nothing asserts or aborts. Invalid arguments are
 * rejected on the host before any HIP call, so an error never leaves work
 * queued. attn_varlen_last_error() gives a message for the calling thread.
 */
#ifndef ATTN_VARLEN_H
#define ATTN_VARLEN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_VARLEN_OK 0
#define ATTN_VARLEN_ENULL (-1)        /* a required pointer is NULL */
#define ATTN_VARLEN_EINVAL (-2)       /* bad count, stride, scale or overlapping output */
#define ATTN_VARLEN_EUNSUPPORTED (-3) /* head_dim not in {64, 96, 128}, stride over limit, or one
                                         segment needing more tiles than a launch holds (2^23 - 1) */
#define ATTN_VARLEN_EALIGN (-4)       /* pointer not 16-byte aligned / stride not a multiple of 8 */
#define ATTN_VARLEN_ECU (-5)          /* cu_seqlens: cu[0] != 0, decreasing, or past the token extents */
#define ATTN_VARLEN_EMAXSEQ (-6)      /* a segment is longer than max_seqlen_q / max_seqlen_k */
#define ATTN_VARLEN_EHIP (-7)         /* HIP runtime or launch failure */

/* Largest token-row stride accepted, in elements (8 MiB rows). */
#define ATTN_VARLEN_MAX_ROW_STRIDE (1LL << 22)

/*
 * Tensor layout. Strides are in ELEMENTS; the innermost (D) stride is always
 * 1. The token extents let the library refuse cu_seqlens that would index
 * past the caller's buffers.
 */
typedef struct attn_varlen_layout {
    int64_t q_row, q_head;
    int64_t k_row, k_head;
    int64_t v_row, v_head;
    int64_t o_row, o_head;
    int64_t lse_head; /* lse[h*lse_head + i]; 0 selects q_tokens */
    int64_t q_tokens; /* token rows addressable in q and out; cu_q[B] <= q_tokens */
    int64_t k_tokens; /* token rows addressable in k and v; cu_k[B] <= k_tokens */
} attn_varlen_layout;

/*
 * Varlen attention forward with cu_seqlens in DEVICE memory (int32, B+1
 * entries each), the calling form of flash_attn_varlen_func on both FA4
 * pages. The library copies the 2*(B+1) integers to the host on `stream` and
 * waits for them (the one synchronisation of the call), checks them, plans an
 * exact grid (one workgroup per (segment, query block, head) tile; no spare
 * blocks, cf. the over-provisioned SingleTileVarlenScheduler grid of the SM120
 * page's "Interpretation") and launches.
 *
 *   q, k, v        bf16 device pointers, 16-byte aligned (q/out may be NULL
 *                  when q_tokens == 0, k/v when k_tokens == 0).
 *   cu_seqlens_q/k int32 device arrays of num_segments+1 cumulative offsets.
 *   num_segments   B >= 0 (B == 0 is a no-op).
 *   num_heads      H >= 1; head_dim D in {64, 96, 128}.
 *   max_seqlen_q/k upper bounds on segment lengths (checked, never trusted).
 *   layout         element strides and token extents (attn_varlen_layout);
 *                  head strides >= 0, row strides in [1,
 *                  ATTN_VARLEN_MAX_ROW_STRIDE], all multiples of 8; out must
 *                  not overlap itself; lse_head >= cu_q[B] when H > 1.
 *   softmax_scale  finite and > 0 (1/sqrt(D) in the pages' configurations).
 *   out            bf16 device pointer, [total_q, H, D] under o_row/o_head.
 *   lse            fp32 device pointer or NULL (no LSE written).
 *   stream         hipStream_t, or NULL for the null stream.
 * Query rows of a segment with no keys get O = 0 and LSE = -inf.
 */
int32_t attn_varlen_fwd(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t num_segments, int32_t num_heads, int32_t head_dim,
                        int32_t max_seqlen_q, int32_t max_seqlen_k,
                        const attn_varlen_layout* layout, float softmax_scale,
                        void* out, float* lse, void* stream);

/*
 * Same operation with cu_seqlens in HOST memory: no device-to-host copy and
 * no synchronisation, so the call only enqueues work on `stream`. The host
 * arrays are read during the call and not kept.
 */
int32_t attn_varlen_fwd_hostcu(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q_host,
                               const int32_t* cu_seqlens_k_host, int32_t num_segments,
                               int32_t num_heads, int32_t head_dim, int32_t max_seqlen_q,
                               int32_t max_seqlen_k, const attn_varlen_layout* layout,
                               float softmax_scale, void* out, float* lse, void* stream);

/*
 * Argument check of attn_varlen_fwd_hostcu without any HIP call: returns the
 * code that call would return before launching. Pointers are only checked
 * for NULL and alignment, never dereferenced (cu arrays are host arrays).
 * The check refuses what the SM120 page's faults come from ("compute-sanitizer
 * memcheck findings", "Interpretation"): cu_seqlens that do not start at 0,
 * decrease, exceed max_seqlen_q/k or index past q_tokens/k_tokens, and
 * strides that would make out overlap itself or exceed the per-tile 32-bit
 * lane offsets (row stride <= ATTN_VARLEN_MAX_ROW_STRIDE); any other error
 * of the call is a HIP runtime failure (ATTN_VARLEN_EHIP).
 */
int32_t attn_varlen_validate(const void* q, const void* k, const void* v,
                             const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
                             int32_t num_segments, int32_t num_heads, int32_t head_dim,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             const attn_varlen_layout* layout, float softmax_scale,
                             const void* out, const float* lse);

/*
 * Query rows per tile (BM) of the general configuration for head_dim (the
 * one used when max_seqlen_k exceeds attn_varlen_one_stage_keys()), or
 * ATTN_VARLEN_EUNSUPPORTED.
 */
int32_t attn_varlen_block_m(int32_t head_dim);

/*
 * Query rows per tile the bf16 forward uses for a call with this
 * max_seqlen_k. Short key segments are the HBM-bound regime, where a tile
 * has little K/V to stream, so the forward switches to smaller workgroups
 * (128 query rows) that share a CU in pairs and overlap each other's loads:
 *   max_seqlen_k <= attn_varlen_one_stage_keys() (128): one K/V stage per
 *     tile, LDS for that stage only;
 *   max_seqlen_k <= attn_varlen_short_stage_keys() (512): 64-key stages in
 *     smaller LDS rings;
 *   longer: the general configuration, attn_varlen_block_m(head_dim).
 * All three give bit-identical results. The choice follows the caller's
 * max_seqlen_k, which every entry point validates against the segments (on
 * the host, or in the device planner), so it never depends on values the host
 * cannot see. The 8-bit forward always uses the general configuration.
 * Returns ATTN_VARLEN_EUNSUPPORTED for an unsupported head_dim and
 * ATTN_VARLEN_EINVAL for max_seqlen_k < 0.
 */
int32_t attn_varlen_block_m_for(int32_t head_dim, int32_t max_seqlen_k);
int32_t attn_varlen_one_stage_keys(void);
int32_t attn_varlen_short_stage_keys(void);

/*
 * Exact tile count H * sum_b ceil(Lq_b / block_m) for host cu_seqlens_q
 * (the per-segment-ceil accounting of the SM120 page's "Interpretation").
 * Returns a negative code on bad arguments (block_m <= 0, H <= 0, bad cu).
 */
int64_t attn_varlen_count_tiles(const int32_t* cu_seqlens_q_host, int32_t num_segments,
                                int32_t num_heads, int32_t block_m);

/*
 * Exact workgroup total of one attn_varlen_fwd / attn_varlen_fwd_hostcu call
 * with these host cu_seqlens_q, num_heads, head_dim and max_seqlen_k:
 * H * sum_b ceil(Lq_b / BM) with BM = attn_varlen_block_m_for(head_dim,
 * max_seqlen_k), summed over the call's launches. This is the per-segment
 * ceil tile accounting of the SM120 page ("Interpretation"), whose launched
 * grid exceeded the valid tile count; here the grid equals this count (15680
 * for that page's cu_seqlens_q at BM = 128 and H = 56). Returns a negative
 * ATTN_VARLEN_E* code on bad arguments (NULL, H <= 0, cu not starting at 0
 * or decreasing, unsupported head_dim, max_seqlen_k < 0, or a segment larger
 * than one launch holds).
 */
int64_t attn_varlen_num_tiles(const int32_t* cu_seqlens_q_host, int32_t num_segments,
                              int32_t num_heads, int32_t head_dim, int32_t max_seqlen_k);

/*
 * Number of kernel launches and workgroups attn_varlen_fwd would use for
 * these host cu_seqlens_q and this max_seqlen_k (which picks the tile
 * height, attn_varlen_block_m_for). Segments are split into launches of at
 * most attn_varlen_segments_per_launch() segments and at most 2^23 - 1 tiles
 * (a launch of 512-thread workgroups stays below 2^32 work-items); each
 * launch's grid is exactly its tile count. Writes the totals to *launches
 * and *workgroups. Returns ATTN_VARLEN_EUNSUPPORTED, as the forward does,
 * when one segment alone needs more tiles than a launch holds.
 */
int32_t attn_varlen_grid_plan(const int32_t* cu_seqlens_q_host, int32_t num_segments,
                              int32_t num_heads, int32_t head_dim, int32_t max_seqlen_k,
                              int64_t* launches, int64_t* workgroups);
int32_t attn_varlen_segments_per_launch(void);

/*
 * Tile decode used by the kernel, exposed for host-side tests: for a launch
 * covering segments with host cu_seqlens_q (B+1 entries, B <= segments per
 * launch), maps workgroup index `wg` to (segment, query block, head).
 * Returns 0, or a negative code when wg is outside the exact grid.
 */
int32_t attn_varlen_decode_tile(const int32_t* cu_seqlens_q_host, int32_t num_segments,
                                int32_t num_heads, int32_t block_m, int64_t wg,
                                int32_t* segment, int32_t* q_block, int32_t* head);

/*
 * Element offset row*row_stride + head*head_stride as the kernel forms it
 * (int64 throughout), exposed so tests can pin it against the wrap values of
 * the _bwd_preprocess page's "Verified sample".
 */
int64_t attn_varlen_element_offset(int64_t row, int64_t row_stride, int64_t head,
                                   int64_t head_stride);

/*
 * Message for the last non-zero return on the calling thread ("" if none).
 * Every entry point reports failure by a code instead of the assertion abort
 * of the ffpa-attn PR #387 page ("Problem": a TMA descriptor assertion ends
 * the process); this gives the reason in words.
 */
const char* attn_varlen_last_error(void);

/*
 * ---- Options: causal masking -------------------------------------------
 *
 * ATTN_VARLEN_CAUSAL: query row r of a segment (0-based within the segment,
 * Lq query and Lk key rows) sees only the keys j <= r + Lk - Lq of that
 * segment, the causal mask aligned to the bottom-right corner of the Lq x Lk
 * score matrix as in the flash-attention interfaces. The pages call
 * flash_attn_varlen_func with causal=False only ("[FA4] cute varlen backward:
 * int32 overflow in _bwd_preprocess ...", repro script), so the alignment is
 * the library's reading. A query row that sees no key (r + Lk - Lq < 0)
 * gets O = 0 and LSE = -inf. Any other bit of `flags` is ATTN_VARLEN_EINVAL.
 */
#define ATTN_VARLEN_CAUSAL 1u

/* attn_varlen_fwd with option flags (flags == 0 is attn_varlen_fwd). */
int32_t attn_varlen_fwd_ex(const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t num_segments, int32_t num_heads, int32_t head_dim,
                           int32_t max_seqlen_q, int32_t max_seqlen_k,
                           const attn_varlen_layout* layout, float softmax_scale, uint32_t flags,
                           void* out, float* lse, void* stream);

/* attn_varlen_fwd_hostcu with option flags. */
int32_t attn_varlen_fwd_hostcu_ex(const void* q, const void* k, const void* v,
                                  const int32_t* cu_seqlens_q_host,
                                  const int32_t* cu_seqlens_k_host, int32_t num_segments,
                                  int32_t num_heads, int32_t head_dim, int32_t max_seqlen_q,
                                  int32_t max_seqlen_k, const attn_varlen_layout* layout,
                                  float softmax_scale, uint32_t flags, void* out, float* lse,
                                  void* stream);

/* attn_varlen_validate with option flags. */
int32_t attn_varlen_validate_ex(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q_host, const int32_t* cu_seqlens_k_host,
                                int32_t num_segments, int32_t num_heads, int32_t head_dim,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                const attn_varlen_layout* layout, float softmax_scale,
                                uint32_t flags, const void* out, const float* lse);

/*
 * ---- Batched dense form ---------------------------------------------------
 *
 * The batched call form flash_attn_func on [W, S, H, D] views, which the
 * "[FA4][SM120] flash_attn_varlen_func ... illegal memory access at >=4 varlen
 * segments" page exercises next to the varlen form in its synthetic sweep
 * ("What rules things out"). It is
 * the varlen operation with W segments of seqlen_q query rows and seqlen_k
 * key rows each; batch b of q/k/v/out is that segment.
 *
 * Layout (strides in ELEMENTS, D contiguous): q[b, s, h, :] at
 * b*q_batch + s*q_row + h*q_head; k, v, out likewise; lse is fp32 [W, H, Sq]:
 * element (b, h, s) at b*lse_batch + h*lse_head + s. Row and batch strides are
 * multiples of 8 elements, row strides at most ATTN_VARLEN_MAX_ROW_STRIDE;
 * out and lse must not overlap themselves; W * seqlen_q and W * seqlen_k
 * must stay below 2^31. No cu_seqlens and no device-to-host copy: the call
 * only enqueues work on `stream`. flags: 0 or ATTN_VARLEN_CAUSAL.
 */
typedef struct attn_batched_layout {
    int64_t q_batch, q_row, q_head;
    int64_t k_batch, k_row, k_head;
    int64_t v_batch, v_row, v_head;
    int64_t o_batch, o_row, o_head;
    int64_t lse_batch, lse_head; /* lse[b*lse_batch + h*lse_head + s] */
} attn_batched_layout;

int32_t attn_fwd_batched(const void* q, const void* k, const void* v, int32_t batch,
                         int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads, int32_t head_dim,
                         const attn_batched_layout* layout, float softmax_scale, uint32_t flags,
                         void* out, float* lse, void* stream);

/* Argument check of attn_fwd_batched without any HIP call. */
int32_t attn_fwd_batched_validate(const void* q, const void* k, const void* v, int32_t batch,
                                  int32_t seqlen_q, int32_t seqlen_k, int32_t num_heads,
                                  int32_t head_dim, const attn_batched_layout* layout,
                                  float softmax_scale, uint32_t flags, const void* out,
                                  const float* lse);

/*
 * ---- Sync-free forward (device planner) ------------------------------------
 *
 * attn_varlen_fwd with device cu_seqlens and NO host synchronisation: the
 * call enqueues two kernels on `stream` and returns. Why: the FA4 SM120 page
 * (its opening motivation) values the kernel most for small inputs, where a
 * per-call device-to-host read-back of cu_seqlens costs as much as the
 * attention itself, and a call without host waits can be captured in a HIP
 * graph.
 *   1. A one-workgroup planner kernel checks cu_seqlens on the device (start
 *      at 0, non-decreasing, segments within max_seqlen_q/k, ends within
 *      q_tokens/k_tokens) and writes the tile prefix into `workspace`.
 *   2. The attention kernel is launched on a grid sized from host-known values
 *      only: at most H * min(ceil((q_tokens + B*(BM-1)) / BM), B*ceil(max_seqlen_q
 *      / BM)) tiles exist (the first term is the SM120 page's grid formula,
 *      "Interpretation"), capped at 8192 workgroups (a multiple of 8). Each
 *      workgroup first reads the planner's status and real tile count, forms
 *      no address for any tile at or past that count (the page's suggested
 *      fix: gate the tile prologue on validity), and loops over tiles
 *      w, w + grid, ... when the count exceeds the grid. One launch serves any
 *      number of segments.
 * Arguments as attn_varlen_fwd_ex, plus:
 *   workspace        device buffer of attn_varlen_async_workspace_bytes(B)
 *                    bytes, 16-byte aligned, owned by the caller; overwritten
 *                    by every call (calls that share one workspace must be
 *                    ordered on one stream).
 *   workspace_bytes  its size.
 * Host-side argument errors are returned as usual. Errors in the cu_seqlens
 * VALUES cannot be returned (the host never sees them): the planner stores
 * ATTN_VARLEN_ECU / ATTN_VARLEN_EMAXSEQ / ATTN_VARLEN_EUNSUPPORTED (tile count
 * >= 2^31) in the workspace's first int32 word, 0 when valid, and the
 * attention kernel then writes nothing. attn_varlen_async_status reads it.
 * Since total_q is unknown on the host, out must not overlap itself over
 * q_tokens rows and a non-zero lse_head must be >= q_tokens when H > 1.
 */
int64_t attn_varlen_async_workspace_bytes(int32_t num_segments);

int32_t attn_varlen_fwd_async(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t num_segments, int32_t num_heads, int32_t head_dim,
                              int32_t max_seqlen_q, int32_t max_seqlen_k,
                              const attn_varlen_layout* layout, float softmax_scale, uint32_t flags,
                              void* workspace, int64_t workspace_bytes, void* out, float* lse,
                              void* stream);

/*
 * attn_varlen_fwd_async for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The caller passes inputs and outputs only; the plan and status
 * words that attn_varlen_fwd_async keeps in the caller's workspace live in a
 * static device array of the library instead (about 256 KiB, one copy per
 * GPU, held until the process ends), whose device address is looked up once
 * per GPU on the first call with that GPU current. The call allocates
 * nothing (no hipMalloc, no library allocation).
 *   num_segments  at most 65536 (the static plan's size); more is
 *                 ATTN_VARLEN_EUNSUPPORTED, returned before any HIP call.
 *   plan          if non-NULL, receives the device address of this GPU's
 *                 static plan (NULL when nothing was enqueued, e.g. B == 0);
 *                 pass it to attn_varlen_async_status to read the call's
 *                 status word once `stream` has reached it.
 * Every call on one GPU uses that GPU's single static plan, and each call's
 * planner rewrites every plan word the call reads (nothing needs clearing).
 * Calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) race on the plan and must not be issued; calls
 * ordered on one stream are safe. Other arguments, results and errors as in
 * attn_varlen_fwd_async.
 */
int32_t attn_varlen_fwd_async_noalloc(const void* q, const void* k, const void* v,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      int32_t num_segments, int32_t num_heads, int32_t head_dim,
                                      int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      const attn_varlen_layout* layout, float softmax_scale,
                                      uint32_t flags, void* out, float* lse, void* stream,
                                      const void** plan);

/* Copy the workspace's status word to *status (waits for `stream`). */
int32_t attn_varlen_async_status(const void* workspace, void* stream, int32_t* status);

/* Workgroups attn_varlen_fwd_async launches for these host-known values. */
int32_t attn_varlen_async_grid(int64_t q_tokens, int32_t num_segments, int32_t num_heads,
                               int32_t head_dim, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int64_t* workgroups);

/*
 * ---- Low-precision forward (8-bit score product) ---------------------------
 *
 * The CDNA4 counterpart of the quantized forward of the "ffpa-attn PR #387"
 * page (its NVFP4 path; "Verification": cos ~0.982 against SDPA, the
 * quantization error), with every size that scales with the sequence length
 * in 64-bit arithmetic (that page's "Fix"). Steps, all on `stream`:
 *   1. per head h: amax_q[h] = max |q[i,h,d]| over rows [0, cu_q[B]), amax_k
 *      likewise over [0, cu_k[B]);
 *   2. codes = E4M3(x * (448 / amax)) (fp32 product, round to nearest even,
 *      OCP E4M3FN), packed [rows, H, D] in the workspace;
 *   3. the forward with S = (codes_q . codes_k) * amax_q/448 * amax_k/448 on
 *      the depth-64 8-bit MFMA; softmax, P (bf16) and P.V (bf16 V) as in
 *      attn_varlen_fwd. Outputs have the same meaning and layout.
 * head_dim 64 or 128 (else ATTN_VARLEN_EUNSUPPORTED); other arguments and
 * errors as attn_varlen_fwd_ex / attn_varlen_fwd_hostcu_ex, plus
 *   workspace        caller-owned device buffer of
 *                    attn_varlen_fp8_workspace_bytes(cu_q[B], cu_k[B], H, D)
 *                    bytes, 256-byte aligned: amax words (2*H uint32, fp32
 *                    bits: q heads, then k heads) at offset 0, then the q and
 *                    k codes at the offsets attn_varlen_fp8_workspace_offsets
 *                    reports. Overwritten by every call.
 */
int64_t attn_varlen_fp8_workspace_bytes(int64_t total_q, int64_t total_k, int32_t num_heads,
                                        int32_t head_dim);
int32_t attn_varlen_fp8_workspace_offsets(int64_t total_q, int64_t total_k, int32_t num_heads,
                                          int32_t head_dim, int64_t* q8_offset, int64_t* k8_offset);

int32_t attn_varlen_fwd_fp8(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t num_segments, int32_t num_heads, int32_t head_dim,
                            int32_t max_seqlen_q, int32_t max_seqlen_k,
                            const attn_varlen_layout* layout, float softmax_scale, uint32_t flags,
                            void* workspace, int64_t workspace_bytes, void* out, float* lse,
                            void* stream);

int32_t attn_varlen_fwd_fp8_hostcu(const void* q, const void* k, const void* v,
                                   const int32_t* cu_seqlens_q_host,
                                   const int32_t* cu_seqlens_k_host, int32_t num_segments,
                                   int32_t num_heads, int32_t head_dim, int32_t max_seqlen_q,
                                   int32_t max_seqlen_k, const attn_varlen_layout* layout,
                                   float softmax_scale, uint32_t flags, void* workspace,
                                   int64_t workspace_bytes, void* out, float* lse, void* stream);

/*
 * ---- Backward -------------------------------------------------------------
 *
 * Gradients of the varlen forward above for an upstream gradient
 * dout = dL/dO: the backward of flash_attn_varlen_func on the "[FA4] cute
 * varlen backward: int32 overflow in _bwd_preprocess ..." page ("Summary";
 * its failing case is a dout view [410923, 16, 96] with row stride 9728 over
 * cu_seqlens [0, 225304, 410923], "Verified sample"). With
 * P[i,j] = exp(scale * Q[i].K[j] - LSE[i]) over the keys j row i sees (its
 * segment's, or with ATTN_VARLEN_CAUSAL the same prefix as the forward), per
 * head h:
 *     D[h,i]  = sum_d out[i,h,d] * dout[i,h,d]            (preprocessing pass)
 *     dS[i,j] = P[i,j] * (dout[i,h,:] . V[j,h,:] - D[h,i])
 *     dQ[i]   = scale * sum_j dS[i,j] K[j],   dK[j] = scale * sum_i dS[i,j] Q[i]
 *     dV[j]   = sum_i P[i,j] dout[i]
 * The page names the preprocessing kernel but not its formula; D above is
 * the library's reading of a per-row reduction over dout and out. out and
 * lse must be the forward's outputs for the same q, k, v, scale and flags.
 * Every gradient element is written by one wave exactly once (no atomics),
 * so results are bitwise reproducible run to run. Rows that see no key get
 * dQ = 0; keys no row sees get dK = dV = 0.
 *
 * Layout (strides in ELEMENTS, D contiguous, every offset formed in int64):
 * q, out, dout, dq: [total_q, H, D] under their own row/head strides; k, v,
 * dk, dv: [total_k, H, D]; lse and delta: fp32, element (h, i) at
 * [h*lse_head + i] / [h*delta_head + i]. Row strides in [1,
 * ATTN_VARLEN_MAX_ROW_STRIDE], head strides >= 0, all multiples of 8; bf16
 * pointers 16-byte aligned, fp32 pointers 4-byte aligned; dq, dk and dv must
 * not overlap themselves; lse_head and delta_head >= cu_q[B] when H > 1.
 */
typedef struct attn_varlen_bwd_layout {
    int64_t q_row, q_head;
    int64_t k_row, k_head;
    int64_t v_row, v_head;
    int64_t o_row, o_head;
    int64_t do_row, do_head;
    int64_t dq_row, dq_head;
    int64_t dk_row, dk_head;
    int64_t dv_row, dv_head;
    int64_t lse_head;   /* lse[h*lse_head + i]; 0 selects q_tokens */
    int64_t delta_head; /* delta[h*delta_head + i]; 0 selects q_tokens */
    int64_t q_tokens;   /* rows addressable in q, out, dout, dq; cu_q[B] <= q_tokens */
    int64_t k_tokens;   /* rows addressable in k, v, dk, dv; cu_k[B] <= k_tokens */
} attn_varlen_bwd_layout;

/*
 * Preprocessing pass alone: delta[h*delta_head + i] = sum_d out[i,h,d] *
 * dout[i,h,d] (fp32) for rows i in [0, rows) and every head, reading out
 * and dout under their own strides (the page's dout view: row stride 9728).
 * rows >= 0 (0 is a no-op); strides and alignment as in the layout above;
 * delta_head >= rows when num_heads > 1. Enqueues one kernel on `stream`.
 */
int32_t attn_varlen_bwd_preprocess(const void* out, const void* dout, int64_t rows,
                                   int32_t num_heads, int32_t head_dim, int64_t o_row,
                                   int64_t o_head, int64_t do_row, int64_t do_head, float* delta,
                                   int64_t delta_head, void* stream);

/*
 * Full backward with cu_seqlens in DEVICE memory (copied to the host and
 * waited for, as in attn_varlen_fwd): the preprocessing pass into `delta`,
 * then the dK/dV and dQ kernels, all on `stream`.
 *   q, k, v, out, dout, lse  the forward's inputs and outputs and the
 *                            upstream gradient (read only).
 *   delta                    fp32 workspace [H, >= total_q] the call
 *                            overwrites (the caller owns it; it holds D
 *                            afterwards).
 *   dq, dk, dv               bf16 outputs, overwritten on every row of the
 *                            segments; rows outside them are not touched.
 *   flags                    0 or ATTN_VARLEN_CAUSAL (as in the forward).
 * Other arguments and errors as in attn_varlen_fwd.
 */
int32_t attn_varlen_bwd(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t num_segments, int32_t num_heads,
                        int32_t head_dim, int32_t max_seqlen_q, int32_t max_seqlen_k,
                        const attn_varlen_bwd_layout* layout, float softmax_scale,
                        uint32_t flags, float* delta, void* dq, void* dk, void* dv, void* stream);

/* attn_varlen_bwd with cu_seqlens in HOST memory: no copy, no synchronisation. */
int32_t attn_varlen_bwd_hostcu(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse,
                               const int32_t* cu_seqlens_q_host,
                               const int32_t* cu_seqlens_k_host, int32_t num_segments,
                               int32_t num_heads, int32_t head_dim, int32_t max_seqlen_q,
                               int32_t max_seqlen_k, const attn_varlen_bwd_layout* layout,
                               float softmax_scale, uint32_t flags, float* delta, void* dq,
                               void* dk, void* dv, void* stream);

/* Argument check of attn_varlen_bwd_hostcu without any HIP call. */
int32_t attn_varlen_bwd_validate(const void* q, const void* k, const void* v, const void* out,
                                 const void* dout, const float* lse,
                                 const int32_t* cu_seqlens_q_host,
                                 const int32_t* cu_seqlens_k_host, int32_t num_segments,
                                 int32_t num_heads, int32_t head_dim, int32_t max_seqlen_q,
                                 int32_t max_seqlen_k, const attn_varlen_bwd_layout* layout,
                                 float softmax_scale, uint32_t flags, const float* delta,
                                 const void* dq, const void* dk, const void* dv);

/*
 * Workgroups of the three backward kernels for these host cu_seqlens:
 * preprocessing, dK/dV (tiles of keys) and dQ (tiles of query rows), and the
 * number of dK/dV and dQ launches (segments are split as in the forward).
 */
int32_t attn_varlen_bwd_grid_plan(const int32_t* cu_seqlens_q_host,
                                  const int32_t* cu_seqlens_k_host, int32_t num_segments,
                                  int32_t num_heads, int32_t head_dim, int64_t* pre_workgroups,
                                  int64_t* dkdv_workgroups, int64_t* dq_workgroups,
                                  int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_VARLEN_H */
