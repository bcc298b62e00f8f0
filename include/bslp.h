/*
 * bslp.h - C ABI of libbslp, an MI355X (gfx950) block-sparse prefill
 * attention library implementing the FlashPrefill / FlashPrefill V2 hot path:
 *
 *   1. bslp_block_scores   mean-pooled keys/values and fused block scores
 *   2. bslp_select_blocks  max-based threshold + sink/window/recent blocks,
 *                          emitted as a CSR selected-block index
 *   3. bslp_sparse_prefill_attn
 *                          causal block-sparse online-softmax attention over
 *                          the selected blocks, with mean correction for the
 *                          pruned fully-visible blocks and PackGQA rows
 *
 * Sources (page title, section):
 *   "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM
 *   Serving", Sec. 3.1, Sec. 3.2, the PackGQA, FP8, CSR, paged-KV and
 *   integration paragraphs; "FlashPrefill: Instantaneous Pattern Discovery
 *   and Thresholding for Ultra-Fast Long-Context Prefilling" (summary page),
 *   method-steps section.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller allocates and owns every buffer.  The library never
 *   allocates, frees or keeps a pointer after a call returns.  Device pointers
 *   must stay valid until the work enqueued on `stream` has finished.
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  All work is
 *   enqueued on it; no call synchronises the host or reads device memory back.
 * Errors: every argument is validated on the host before anything is
 *   launched; a call that returns an error has enqueued nothing.  Launch
 *   failures return BSLP_ERR_HIP.  bslp_last_error() gives a thread-local text
 *   for the last failing call of the calling thread.  No exception crosses
 *   the ABI and there is no global mutable state besides that text.
 * Sequences: requests are packed back to back ("varlen").  Request b has
 *   L_b = kv_seqlens[b] keys at positions 0 .. L_b - 1 and Lq_b = seqlens[b]
 *   queries: the last Lq_b positions, off_b = L_b - Lq_b .. L_b - 1 (a chunk
 *   of a chunked prefill, FlashPrefill V2 integration paragraph; off_b = 0
 *   for a whole prompt, when kv_seqlens is NULL).  Its queries own Q / O rows
 *   (and LSE columns) [qstart_b, qstart_b + Lq_b), qstart_b = sum_{b'<b}
 *   Lq_b'; its keys own contiguous K / V rows [kstart_b, kstart_b + L_b),
 *   kstart_b = sum_{b'<b} L_b'.
 * Blocks: key block J of request b covers positions [J*B, min((J+1)*B, L_b));
 *   N_b = ceil(L_b / B).  Query tile I covers the query positions inside
 *   block I, for the g = Hq/Hkv query heads of one KV head (PackGQA rows,
 *   FlashPrefill V2 PackGQA paragraph); the tiles that hold a query are
 *   I = i0_b .. N_b - 1 with i0_b = floor(off_b / B) (none if Lq_b = 0), and
 *   one selection is made per (request, KV head, tile), re-run per chunk.
 * Segments: s(b, h, I) = seg_base_b + h*(N_b - i0_b) + I - i0_b with
 *   seg_base_b = sum_{b'<b} Hkv*(N_b' - i0_b').  Score rows: row (b, h, I)
 *   has I+1 floats at score_base_b + h*T_b + I(I+1)/2 - i0_b(i0_b+1)/2, with
 *   T_b = N_b(N_b+1)/2 - i0_b(i0_b+1)/2 and score_base_b = sum_{b'<b} Hkv*T_b'.
 *   Pooled rows: block J of request b is pooled row pool_base_b + J,
 *   pool_base_b = sum_{b'<b} N_b' (every key block is pooled).
 */
#ifndef BSLP_H
#define BSLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bslp_status {
  BSLP_OK = 0,
  BSLP_ERR_INVALID_ARG = 1, /* null pointer, inconsistent shape, bad value  */
  BSLP_ERR_UNSUPPORTED = 2, /* valid but not built (head_dim, block, limits) */
  BSLP_ERR_HIP = 3,         /* a HIP launch or runtime call failed          */
  BSLP_ERR_WORKSPACE = 4    /* workspace NULL, too small or misaligned      */
} bslp_status;

typedef enum bslp_dtype {
  BSLP_F32 = 0,      /* float32 Q/K/V, float32 output                       */
  BSLP_BF16 = 1,     /* bfloat16 Q/K/V, bfloat16 output                     */
  BSLP_FP8_E4M3 = 2  /* OCP e4m3fn codes (uint8) with one float scale per
                        tensor (FlashPrefill V2, FP8 paragraph); bf16 output */
} bslp_dtype;

/* Problem descriptor; read during the call only. */
typedef struct bslp_problem {
  int32_t dtype;          /* bslp_dtype                                      */
  int32_t num_heads_q;    /* Hq                                              */
  int32_t num_heads_kv;   /* Hkv; Hq % Hkv == 0, g = Hq / Hkv <= 16          */
  int32_t head_dim;       /* d: 64 or 128                                    */
  int32_t block_size;     /* B: 64 or 128                                    */
  float softmax_scale;    /* multiplies q.k (normally 1/sqrt(d)), > 0        */
  float q_scale;          /* per-tensor dequantisation scales for fp8; each  */
  float k_scale;          /*   fp8 element x decodes to code(x) * scale.     */
  float v_scale;          /*   Must be 1 for f32 / bf16.                     */
  int32_t num_seqs;       /* 1 .. 64                                         */
  const int32_t* seqlens; /* HOST array [num_seqs]: queries Lq_b >= 0        */
  /* Paged K/V (FlashPrefill V2, paged-KV paragraph): when page_table is not
   * NULL, key/value token j of request b lives at physical row
   * page_table[b * max_pages_per_seq + j / page_size] * page_size
   * + j % page_size of the K/V arrays.  page_size is a power of two.
   * Entries must address rows inside the caller's K/V arrays; they are not
   * range-checked on the device. */
  const int32_t* page_table; /* DEVICE [num_seqs, max_pages_per_seq] or NULL */
  int32_t page_size;
  int32_t max_pages_per_seq;
  /* KV splitting of the attention ("FlashPrefill V2", CSR paragraph, Eq. 18,
   * and the scheduling paragraph after it: a work unit's
   * selected blocks are cut into contiguous shares balanced by count, each
   * run by its own workgroup, and the partial results are merged through
   * their log-sum-exp).  1 = never, 2..16 = that many splits at most,
   * 0 = automatic: with units = sum_b (N_b - i0_b) * Hkv * ceil(g B / R)
   * work units of R = 256, 128 or 64 packed rows (the largest not above
   * g B), a launch of fewer than 512 units in which some request has at
   * least 16 blocks allows min(4, ceil(512 / units)) splits, any other
   * launch none.  A segment with n selected blocks then uses
   * max(1, min(allowed, steps / 24)) splits, steps = n B / 64 plus
   * ceil(I / 64) when mean correction is on and I > 0; split u of U takes
   * CSR positions [u n / U, (u + 1) n / U) and the correction chunks
   * u, u + U, ... .  bf16 / fp8 only; the float32 path never splits.  It
   * changes bslp_sizes.workspace_bytes. */
  int32_t kv_splits;
  /* fp8 only: DEVICE float[3] = (q_scale, k_scale, v_scale), as written by
   * bslp_quantize_e4m3, or NULL to use the host floats above (then ignored).
   * Read by the kernels, so no host synchronisation is needed between the
   * quantisation and the prefill. */
  const float* scales_dev;
  /* HOST array [num_seqs]: keys L_b >= seqlens[b], N_b <= 16384; NULL means
   * L_b = seqlens[b] (self prefill of whole prompts). */
  const int32_t* kv_seqlens;
  /* Layout of V (FlashPrefill V2, FP8 paragraph: the fp8 P~V product takes
   * V with the keys along the contiguous dimension).
   *   BSLP_V_ROWS (0): like K, [kv tokens, Hkv, d] (or [pages * page_size,
   *     Hkv, d] when paged);
   *   BSLP_V_DMAJOR (1), fp8 only: [Hkv, d, kv tokens] contiguous, or
   *     [pages, Hkv, d, page_size] paged with page_size >= 64; token j of
   *     request b is column kv_start_b + j (contiguous) or column j %
   *     page_size of its page.  Every V reader (pooling, the quantised
   *     pooled values, attention) takes this layout; outputs do not change.
   * Anything else is BSLP_ERR_INVALID_ARG; d-major V with a non-fp8 dtype or
   * pages below 64 tokens is BSLP_ERR_UNSUPPORTED. */
  int32_t v_layout;
} bslp_problem;

enum { BSLP_V_ROWS = 0, BSLP_V_DMAJOR = 1 };

/* Selection hyper-parameters (FlashPrefill V2, Sec. 3.1 and Sec. 4: alpha and
 * the sink/window sizes are user settings).  Counts are in blocks:
 *   sink   = blocks 0 .. sink_blocks-1,
 *   recent = the recent_blocks blocks ending at the diagonal block I,
 *   window = the window_blocks blocks just before the recent ones,
 * all clipped to 0 .. I. */
typedef struct bslp_select_params {
  float alpha;             /* thresh_I = alpha * max_J Score_IJ, alpha >= 0  */
  int32_t sink_blocks;     /* >= 0 */
  int32_t window_blocks;   /* >= 0 */
  int32_t recent_blocks;   /* >= 0 */
  int32_t mean_correction; /* 0 or 1 */
} bslp_select_params;

/* Buffer sizes implied by a problem. */
typedef struct bslp_sizes {
  int64_t total_tokens; /* T = sum Lq_b: rows of Q and O, columns of LSE      */
  int64_t pooled_rows;  /* sum N_b: rows of kbar / vbar                       */
  int64_t score_elems;  /* sum Hkv T_b: scores and idx capacity               */
  int64_t num_segments; /* sum Hkv (N_b - i0_b): entries of counts (cu: +1)   */
  int64_t workspace_bytes; /* device scratch bslp_sparse_prefill_attn needs     */
  int64_t kv_tokens;    /* sum L_b: rows of contiguous K and V                */
} bslp_sizes;

/* Validates `problem` and fills `out`.  Host only; no HIP call. */
bslp_status bslp_get_sizes(const bslp_problem* problem, bslp_sizes* out);

/* The workspace bslp_sparse_prefill_attn needs for `problem`, in bytes (the
 * workspace_bytes of bslp_get_sizes); 0 when the problem is invalid, with the
 * reason in bslp_last_error().  Host only; no HIP call.  The workspace is
 * reused by every layer of a forward pass (the pages build per-forward
 * metadata once, with no allocator round trip), so one query per shape is
 * enough. */
size_t bslp_workspace_bytes(const bslp_problem* problem);

/* Stage 1: pooled means and block scores.
 *
 * Pooling (FlashPrefill V2, Sec. 3.1; pooled values for Sec. 3.2):
 *   kbar[pool_base_b + J, h, :] = mean of k over the tokens of block J,
 *   vbar likewise; float32 [pooled_rows, Hkv, d].  For fp8 the means are of
 *   the dequantised values (code * k_scale).
 * Scores (FlashPrefill summary page, method steps; V2 Sec. 3.1): for every
 *   (b, h, I) and J <= I, with s_rJ = softmax_scale * q_r . kbar_J over the
 *   tile's g*|tile| rows r (block-causal, no token mask in the diagonal
 *   block), M_I = max_{r, J<=I} s_rJ, S'_IJ = sum_r exp(s_rJ - M_I),
 *   Score_IJ = S'_IJ / sum_{K<=I} S'_IK, written to scores (float32 rows as
 *   described above).  Accuracy: float32 inputs accumulate the logits in
 *   float64 on the vector ALUs.  bf16 / fp8 inputs run on the matrix cores:
 *   q is exact in bf16 and kbar is split into two bf16 terms (to within
 *   2^-18 of itself), products are exact and the accumulation is float32;
 *   the scores carry a relative error below 1e-3 (of order 1e-5 on the 64K
 *   and 128K workloads), which bslp_select_blocks absorbs by deciding the
 *   blocks near the threshold exactly.
 *
 * q: [T, Hq, d] in the problem dtype.  k, v: [T, Hkv, d], or physical rows
 * [*, Hkv, d] through the page table.  All device pointers. */
bslp_status bslp_block_scores(const bslp_problem* problem, const void* q, const void* k,
                              const void* v, float* kbar, float* vbar, float* scores,
                              void* stream);

/* The two halves of bslp_block_scores, for callers that time or overlap
 * them separately; together they enqueue exactly the launches of
 * bslp_block_scores.
 * bslp_pool_kv: the pooled means kbar, vbar from k, v (as above).
 * bslp_score_blocks: the score rows from q and the kbar of bslp_pool_kv for
 *   the same problem.  Errors as bslp_block_scores. */
bslp_status bslp_pool_kv(const bslp_problem* problem, const void* k, const void* v, float* kbar,
                         float* vbar, void* stream);
bslp_status bslp_score_blocks(const bslp_problem* problem, const void* q, const float* kbar,
                              float* scores, void* stream);

/* Stage 2: selection (FlashPrefill V2, Sec. 3.1 threshold paragraph and the
 * CSR paragraph; threshold formula printed on the FlashPrefill summary page).
 *   thresh_I = alpha * max_{J<=I} Score_IJ;
 *   Sel_I = {J <= I : Score_IJ >= thresh_I} u sink u window u recent.
 * Outputs (device, int32):
 *   counts[s] = |Sel| of segment s                        [num_segments]
 *   cu[s]     = sum_{s'<s} counts[s'], cu[num_segments] = total
 *                                                         [num_segments + 1]
 *   idx[cu[s] .. cu[s+1]) = Sel of segment s, ascending  [score_elems capacity]
 * alpha = 0 selects every causal block (dense attention).
 * Exactness: the scores carry a relative error below 1e-3; every block
 * whose score lies within 2e-3 (relative) of thresh_I is re-decided exactly
 * in float64 from q and kbar (the comparison E_J >= alpha max_K E_K of block
 * energies E_J = sum_r exp(s_rJ - m), the maximum taken over the blocks
 * within 2e-3 of the largest score), so the selection is the definition's
 * outside a float64-rounding band.  q and kbar are the inputs of stage 1
 * for the same problem (kbar from bslp_block_scores / bslp_pool_kv).
 * scores: read, and borrowed in between: the call's first pass hands the
 * exact decisions to its last pass by negating the scores of the re-decided
 * blocks it drops, and the last pass restores them, so when the call's work
 * on `stream` has completed the buffer holds bitwise what it held before.
 * No other work may read or write scores while the call's work runs. */
bslp_status bslp_select_blocks(const bslp_problem* problem, const bslp_select_params* params,
                               const void* q, const float* kbar, float* scores,
                               int32_t* counts, int32_t* cu, int32_t* idx, void* stream);

/* Stage 3: block-sparse causal attention with mean correction
 * (FlashPrefill V2, Sec. 3.1 last sentence, Sec. 3.2 and Fig. 3, PackGQA and
 * CSR paragraphs).  For query row (i, hq) of tile I, KV head h = hq / g:
 *   exact terms  e_j = softmax_scale * q . k_j for the tokens j <= i of the
 *                blocks in Sel_I (read from cu/idx);
 *   correction   if params->mean_correction: for every J <= I-1 not in Sel_I,
 *                c_J = softmax_scale * q . kbar_J + ln|B_J| with value vbar_J;
 *   O = sum softmax weights * values, LSE = m + ln l (natural log).
 * Walk: each segment's selected blocks are taken from the last to the
 * first, each in 64-key tiles from the highest to the lowest, then the
 * correction terms in chunks of 64 pooled blocks (CSR paragraph; tile
 * configuration paragraph).  bf16 and float32 results depend on it only
 * through rounding.
 * fp8 arithmetic (FP8 paragraph; Tab. 8 paragraph): with c_q, c_k, c_v the
 * per-tensor scales, logits are softmax_scale c_q c_k (Q~ K~^T), computed
 * exactly on the bf16 matrix cores; m is the exact running row maximum of
 * the walk; each probability is rounded to e4m3 as P~ = e4m3(2^8 exp(s - m))
 * (nearest even) and O = c_v (P~ V~) / l with l = sum P~, on the fp8 matrix
 * cores; LSE = m + ln l - 8 ln 2.  The correction terms use the pooled
 * statistics rounded the same way: e4m3 of the exact mean of each block's K
 * (V) codes, computed from k and v themselves (kbar and vbar are not read
 * for fp8).  A probability within about 1e-5 of an e4m3 rounding midpoint
 * may round either way.
 * out: [T, Hq, d], float32 for BSLP_F32 else bfloat16.  lse: float32
 * [Hq, T] or NULL.  A row that sees no key gets O = 0 and LSE = -inf.
 * kbar / vbar / cu / idx are the outputs of stages 1 and 2 for the same
 * problem.  Only params->mean_correction is read.
 * workspace: device scratch of at least bslp_workspace_bytes(problem) bytes,
 * 16-byte aligned, owned by the caller; its contents on entry do not matter
 * and are overwritten (the call keeps bf16 copies of kbar, as hi + lo pairs,
 * and of vbar there; for fp8 the quantised pooled codes; with KV splits the
 * partial results; and the list of work units, one int32 each, with its
 * queue counters, which persistent launches take units from: split
 * launches, and unsplit bf16 ones with at least 16 units per compute unit).
 * A NULL (when bytes are needed), short or misaligned
 * workspace is BSLP_ERR_WORKSPACE, before any launch.  Calls that overlap in
 * time must not share a workspace. */
bslp_status bslp_sparse_prefill_attn(const bslp_problem* problem,
                                     const bslp_select_params* params, const void* q,
                                     const void* k, const void* v, const float* kbar,
                                     const float* vbar, const int32_t* cu, const int32_t* idx,
                                     void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Stage 3 for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, kernels and results as bslp_sparse_prefill_attn, with
 * the workspace replaced by a device array inside the library of
 * BSLP_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the first call on a
 * device until the process ends.  Nothing is allocated or freed by the call.
 * Arguments as bslp_sparse_prefill_attn, without workspace / workspace_bytes.
 * Limits: the workspace bslp_get_sizes reports must fit the array; an
 * automatic KV split count (kv_splits = 0) whose partial results would not
 * fit falls back to no split, and any other overflow returns
 * BSLP_ERR_UNSUPPORTED before anything is enqueued (kv_splits = 1 needs
 * 6 * pooled_rows * Hkv * d bytes: 32 MiB covers 5.4M pooled (block, KV
 * head) rows of 64 dims or 2.7M of 128).  Every call on one GPU shares its
 * array, which keeps the last call's contents (nothing in it needs to start
 * at zero); calls that overlap in time on one GPU race on it and must be
 * serialised by the caller, e.g. by issuing them on one stream. */
#define BSLP_NOALLOC_SCRATCH_BYTES (32u << 20)
bslp_status bslp_sparse_prefill_attn_noalloc(const bslp_problem* problem,
                                             const bslp_select_params* params, const void* q,
                                             const void* k, const void* v, const float* kbar,
                                             const float* vbar, const int32_t* cu,
                                             const int32_t* idx, void* out, float* lse,
                                             void* stream);

/* Dense causal prefill attention on the same kernels, with no index stage:
 * every row attends to all keys j <= i of its request, as a
 * FlashAttention-style dense baseline against which the block-sparse path's
 * speedup is measured ("FlashPrefill V2", Sec. 4 comparisons with dense
 * FlashAttention; its kernel-speed figures).
 *
 * q, k, v, page table, out and lse as in bslp_sparse_prefill_attn (same
 * layouts, dtypes and scales); no pooled means, index or workspace are read.
 * The result equals bslp_sparse_prefill_attn's with every causal block
 * selected and mean correction off, bit for bit: the same blocks are walked
 * in the same order.  Errors: as bslp_sparse_prefill_attn. */
bslp_status bslp_dense_prefill_attn(const bslp_problem* problem, const void* q, const void* k,
                                    const void* v, void* out, float* lse, void* stream);

/* Online per-tensor fp8 quantisation ("FlashPrefill V2", the FP8 paragraph:
 * e4m3 operands, one absmax-derived scale per tensor, computed on the device): with amax = max_i |x_i|, *scale = amax / 448 (1 if amax is 0)
 * and codes[i] = e4m3fn(x_i / *scale), rounded to nearest even, saturated at
 * +-448, sign kept (float32 division, correctly rounded).
 *
 * x: DEVICE, n elements of src_dtype (BSLP_BF16 or BSLP_F32), 16-byte
 * aligned.  codes: DEVICE uint8 [n], 8-byte aligned.  scale: DEVICE float,
 * 4-byte aligned; it also serves as the accumulator of the maximum, so
 * calls that share it must not overlap.  Paged K/V caches are quantised
 * whole: every one of the n elements counts towards amax.  Four launches on
 * `stream`; nothing is synchronised.  Errors: invalid dtype, n < 0, NULL or
 * misaligned pointers (BSLP_ERR_INVALID_ARG, before any launch). */
bslp_status bslp_quantize_e4m3(int32_t src_dtype, const void* x, int64_t n, uint8_t* codes,
                               float* scale, void* stream);

/* Static text for a status code. */
const char* bslp_status_string(bslp_status status);
/* Detail of the calling thread's last failing call ("" if none). */
const char* bslp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BSLP_H */
