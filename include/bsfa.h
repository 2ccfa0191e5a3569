/*
 * bsfa.h - C ABI of libbsfa.so: exact-score-gated block-sparse causal prefill attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation ("Block Sparse Flash Attention", paper notes, Method):
 *   For every batch b, query head h and query block i (query rows [i*Bq, (i+1)*Bq), at
 *   absolute positions P + i*Bq .. with P = kv_seqlen - seqlen, 0 for a whole prefill), the
 *   kernel visits the causally visible key blocks j (columns [j*Bk, (j+1)*Bk)) in ascending
 *   order and computes the exact scaled scores S = Q_i K_j^T * scale of the whole tile (Key
 *   Designs 2).
 *     - Off-diagonal blocks (j < n_off(i) = floor((P + i*Bq)/Bk), wholly before the block's
 *       first row) are gated. ABSOLUTE: keep iff s_max = max over the tile of S >= T_eff(h, i) (Key Designs
 *       2, keep-rule equation; ">=" as in the main text). RELATIVE: keep iff some row r of the
 *       tile has rowmax_j[r] - m[r] >= log_lambda, m the running row max before the block
 *       ("Skipping attention blocks was the easy part", BLASST blog, section "Vote, then skip").
 *       DENSE: keep every block (the gate is compiled out).
 *     - Diagonal-region blocks (n_off(i) <= j < n_end(i)) always run, with the causal mask.
 *     - A kept block updates the online-softmax state (running max m, sum l, accumulator O)
 *       and accumulates P V_j; a skipped block loads no V, adds nothing and leaves m, l and O
 *       untouched (Key Designs 3); it gets no exponentials either, also where the decision is
 *       voted inside the softmax loop (the vote comes before them).
 *     - Output O_i = O / l: attention renormalised over the kept blocks and the diagonal
 *       region (Overall Architecture; Key Designs 3).
 *   T_eff(h, i) = T[budget_slice][h][min(P/Bq + i, t_len - 1)] (the absolute query block):
 *   positions past the calibrated length reuse the last calibrated column (Key Designs 1).
 *   -INFINITY keeps every block.
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory on the current HIP device; the library
 *     allocates nothing and frees nothing. Between calls it keeps only the thread-local error
 *     string and per-device facts it looks up once (the static scratch's address, how many
 *     workgroups of a kernel the device holds at once).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is asynchronous:
 *     results are valid once the caller has synchronised the stream. The library never
 *     synchronises.
 *   - Arguments are validated on the host before anything is enqueued. On any status other
 *     than BSFA_OK and BSFA_ERR_HIP nothing was enqueued and every output is untouched;
 *     bsfa_last_error() then describes the problem. BSFA_ERR_HIP means a launch failed; earlier
 *     launches of the same call (zeroing kept_total or the workspace's counters, FP8 copies,
 *     block means, the gate sweep) may already be enqueued, and the outputs are then
 *     undefined. No C++ exception crosses
 *     the ABI.
 *   - Tensors are indexed [batch][token][head][dim] with element strides given per tensor for
 *     batch, token and head; the dim axis is contiguous. Base pointers and every row
 *     (batch/token/head offset) must be 16-byte aligned.
 */
#ifndef BSFA_H_
#define BSFA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSFA_OK = 0,
  BSFA_ERR_ARG = 1,          /* NULL pointer, negative size, bad enum value */
  BSFA_ERR_SHAPE = 2,        /* heads_q % heads_kv != 0, unsupported head_dim or tile */
  BSFA_ERR_DTYPE = 3,        /* unsupported input or output dtype */
  BSFA_ERR_ALIGN = 4,        /* pointer or stride breaks the 16-byte row alignment */
  BSFA_ERR_TABLE = 5,        /* threshold table missing or its header disagrees with the problem */
  BSFA_ERR_UNSUPPORTED = 6,  /* valid request outside what this library implements */
  BSFA_ERR_HIP = 7           /* the HIP runtime reported an error at launch */
} bsfa_status;

typedef enum {
  BSFA_GATE_DENSE = 0,       /* keep every block: the dense path */
  BSFA_GATE_ABSOLUTE = 1,    /* keep iff s_max >= T_eff(h, i) */
  BSFA_GATE_RELATIVE = 2     /* keep iff max_r(rowmax_j[r] - m[r]) >= log_lambda */
} bsfa_gate_mode;

typedef enum { BSFA_BF16 = 0, BSFA_FP32 = 1, BSFA_FP8_E4M3 = 2 } bsfa_dtype;

/* One causal prefill self-attention call (one layer). */
typedef struct {
  int32_t batch;             /* B >= 0 */
  int32_t seqlen;            /* N >= 0 query tokens; need not be a tile multiple */
  int32_t heads_q;           /* Hq >= 1 */
  int32_t heads_kv;          /* Hkv >= 1, Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv) */
  int32_t head_dim;          /* d: 64 or 128 */
  int32_t block_q;           /* Bq: 64 or 128 (gate tile rows) */
  int32_t block_k;           /* Bk: 64, or 128 with Bq = 128 (gate tile columns). 128-key blocks
                              * (the notes re-tile for other hardware and recalibrate, "Block
                              * Sparse Flash Attention", Loss & Training) are decided by the gate
                              * sweep: DENSE, and ABSOLUTE with a workspace; RELATIVE, ABSOLUTE
                              * without a workspace and bsfa_prefill's debug_block_stat return
                              * BSFA_ERR_UNSUPPORTED for them. Loads and loop steps stay at 64
                              * keys; decisions, kept counts and block statistics are per block. */
  float softmax_scale;       /* > 0, or 0 for 1/sqrt(head_dim); applied to fp32 scores */
  int32_t in_dtype;          /* bsfa_dtype of Q, K, V: BSFA_BF16 */
  int32_t out_dtype;         /* bsfa_dtype of O: BSFA_BF16 or BSFA_FP32 */
  int64_t q_stride[3];       /* element strides of Q for batch, token, head */
  int64_t k_stride[3];       /* element strides of K */
  int64_t v_stride[3];       /* element strides of V */
  int64_t o_stride[3];       /* element strides of O */
  int32_t kv_seqlen;         /* key tokens Nk: 0 means N (a whole prefill); otherwise Nk >= N and
                              * the N query tokens are the last N of the Nk positions (a chunk
                              * after a prefix of P = Nk - N cached keys). Query block i then
                              * starts at absolute row P + i*Bq: the causal mask, the off-diagonal
                              * range and the threshold column (P/Bq + i) use absolute positions,
                              * and the absolute gate needs P % Bq == 0 (thresholds live on the
                              * calibration's tile grid). K and V hold Nk rows. */
  int32_t mean_correction;   /* 0 or 1. 1: every pruned off-diagonal gate block J adds a
                              * zero-order stand-in, |B_J| e^{s_J} vbar_J to the numerator and
                              * |B_J| e^{s_J} to the denominator, with kbar_J, vbar_J the block's
                              * mean key and value, s_J = softmax_scale * q . kbar_J and |B_J| its
                              * keys ("FlashPrefill V2: Block-Sparse Prefill Attention for
                              * Long-Context LLM Serving", mean correction). Needs ABSOLUTE with
                              * a 16-byte-aligned workspace, which then also holds the block means
                              * (bsfa_prefill_workspace_bytes counts them); RELATIVE (whose
                              * decisions read the running max a stand-in would move) and
                              * ABSOLUTE without a workspace return BSFA_ERR_UNSUPPORTED. DENSE
                              * prunes nothing: no effect. */
  int32_t gate_dtype;        /* precision of the absolute gate's scores: BSFA_BF16 (0, the exact
                              * scores) or BSFA_FP8_E4M3: the gate sweep scores E4M3 copies of Q
                              * and K on the FP8 matrix cores (FlashPrefill V2's FP8 path; the
                              * softmax and O still use the exact bf16 scores of the kept
                              * blocks). Q is quantised per (token, head) row and K per (64-key
                              * tile, KV head): scale = amax / 448, code = x * (448 / amax)
                              * rounded to nearest even on the E4M3 grid (fp32); a score is
                              * (q8 . k8) * scale_q * scale_k * softmax_scale. Thresholds must be
                              * calibrated on the same FP8 scores. Needs ABSOLUTE with a
                              * 16-byte-aligned workspace, which then also holds the copies;
                              * RELATIVE returns BSFA_ERR_UNSUPPORTED; DENSE ignores it. */
} bsfa_problem;

/* One layer's threshold table (the offline calibration artifact), fp32 in device memory.
 * T holds n_budgets slices, each [heads_q][t_len] row-major; entries may be +-INFINITY.
 * The header fields record the tile semantics the table was calibrated for and must agree
 * with the problem: a threshold's meaning changes with the model and the tile shape
 * ("Block Sparse Flash Attention", Method > Key Designs 1, last paragraph). */
typedef struct {
  const float* T;            /* device, 4-byte aligned, n_budgets * heads_q * t_len floats */
  int32_t n_budgets;         /* >= 1 */
  int32_t t_len;             /* >= 1 calibrated query blocks; blocks i >= t_len use t_len - 1 */
  int32_t heads_q;           /* must equal problem heads_q */
  int32_t block_q;           /* must equal problem block_q */
  int32_t block_k;           /* must equal problem block_k */
  int32_t head_dim;          /* must equal problem head_dim */
  float softmax_scale;       /* must equal the effective scale within 1e-6 relative */
  const int32_t* budgets;    /* host, n_budgets entries: the budget k (off-diagonal blocks) each
                              * slice was calibrated for, or NULL if unknown; an entry <= 0 also
                              * means unknown. Read during the call only. The library uses it
                              * to predict how many blocks a call keeps (the budget is a target
                              * on the count of kept blocks, "Block Sparse Flash Attention",
                              * Method > Key Designs 1) and so to choose how to run the absolute
                              * gate (see bsfa_prefill's workspace). */
} bsfa_table;

/* Bytes of device workspace bsfa_prefill can use for `gate_mode` (0 for an invalid problem
 * or gate_mode): for DENSE and RELATIVE, 256 bytes that hold a counter from which the
 * workgroups take their (b, h, i) units in turn; for ABSOLUTE, one keep bitmask per (b, h, i) with one bit per 64-key tile,
 * B * Hq * ceil(N/Bq) * ceil(ceil(Nk/64)/64) uint64 words; then, each part starting on a
 * 256-byte boundary: with gate_dtype FP8_E4M3 the E4M3 copies of Q [B][N][Hq][d] and K
 * [B][Nk][Hkv][d] (one byte per element) and their fp32 scales [B][Hq][N] and
 * [B][Hkv][ceil(Nk/64)]; with mean_correction three bf16 arrays [B][Hkv][floor(Nk/Bk)][d]: the
 * block means of K in two parts (high and low bf16) and of V; last, 256 bytes for a counter
 * from which the workgroups of the softmax launch take their (b, h, i) units in turn. */
uint64_t bsfa_prefill_workspace_bytes(const bsfa_problem* p, int32_t gate_mode);

/* Gated causal prefill attention (the method's hot path).
 *   p             problem description (host memory, read during the call only)
 *   Q             device [B][N][Hq][d] bf16;  K, V: device [B][Nk][Hkv][d] bf16
 *   table         threshold table; required for ABSOLUTE, ignored otherwise (may be NULL)
 *   budget_slice  which table slice (0 <= budget_slice < n_budgets) for ABSOLUTE
 *   gate_mode     bsfa_gate_mode
 *   log_lambda    RELATIVE only: ln(lambda); -INFINITY (lambda = 0) never skips
 *   O             device [B][N][Hq][d] in out_dtype, written for every row
 *   kept_counts   device int32 [B][Hq][ceil(N/Bq)] or NULL: number of kept OFF-diagonal
 *                 blocks per (b, h, i); the diagonal region is not counted ("Block Sparse
 *                 Flash Attention", A Worked Example: it does not consume the budget)
 *   kept_total    device uint64 scalar or NULL: sum of kept_counts (zeroed, then accumulated,
 *                 on `stream`)
 *   debug_block_stat  device fp32 [B][Hq][ceil(N/Bq)][ceil(Nk/Bk)] or NULL: per visible block,
 *                 the gate statistic in scaled-score units (ABSOLUTE and DENSE: s_max;
 *                 RELATIVE: max_r(rowmax_j[r] - m[r]) for off-diagonal blocks, s_max for the
 *                 diagonal region). Entries of invisible blocks (j >= n_end(i)) are not written.
 *   workspace     device, 8-byte aligned, or NULL; caller-owned scratch of workspace_bytes
 *                 (its contents on return are unspecified). A softmax launch over every
 *                 block (DENSE, RELATIVE, and ABSOLUTE's one launch below) with a workspace
 *                 holds as many workgroups as stay resident, which take the (b, h, i) units in
 *                 turn from a counter in it; without one each unit runs in a workgroup of its
 *                 own (the same results bit for bit; the first is faster where units differ
 *                 in length, as causal ones do). The absolute gate runs in one of
 *                 two ways with the same results (O, kept counts and statistics bit for bit):
 *                 two launches, a gate sweep that decides every block from its scores alone
 *                 and writes keep masks into the workspace, then a softmax launch that walks
 *                 the kept blocks only; or one launch that decides each block inside the
 *                 softmax loop. Without a workspace the call takes one launch. With a
 *                 workspace of at least bsfa_prefill_workspace_bytes(p, gate_mode) bytes it
 *                 takes two, unless the table records the slice's budget k and either
 *                 sum_i min(n_off(i), k) / sum_i n_off(i) (the share of off-diagonal blocks
 *                 the budget keeps) exceeds 1/2 for this problem — when most blocks are kept
 *                 the second pass over them costs more than deciding inside the loop — or
 *                 the call has fewer than 65536 off-diagonal tiles in all
 *                 (B * Hq * sum_i n_off(i)), where the second launch's fixed costs
 *                 outweigh the work it saves. A
 *                 non-NULL workspace that is too small is an error (BSFA_ERR_ARG). With
 *                 mean_correction, an FP8 gate or block_k = 128 it is required (two launches
 *                 always) and must be 16-byte aligned; a launch before the sweep computes the
 *                 block means, and one the FP8 copies.
 *   stream        hipStream_t
 * The absolute gate supports Nk up to 2097152 (BSFA_ERR_UNSUPPORTED beyond).
 * Returns BSFA_OK or an error status (see the conventions above). */
bsfa_status bsfa_prefill(const bsfa_problem* p, const void* Q, const void* K, const void* V,
                         const bsfa_table* table, int32_t budget_slice, int32_t gate_mode,
                         float log_lambda, void* O, int32_t* kept_counts, uint64_t* kept_total,
                         float* debug_block_stat, void* workspace, uint64_t workspace_bytes,
                         void* stream);

/* bsfa_prefill for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same computation and results as
 * bsfa_prefill with a caller workspace of bsfa_prefill_workspace_bytes(p, gate_mode) bytes, with
 * the absolute gate's workspace (keep masks; with mean_correction also the block means; with
 * an FP8 gate also the FP8 copies) taken from a static 64 MiB device array that the library
 * holds on each device it runs on until the process ends. The call itself allocates and frees
 * nothing; the caller passes inputs and outputs as for bsfa_prefill (arguments of the same
 * names mean the same). The array's device address is looked up on the first call on each
 * device (that call must find the device current, as every call must).
 *   Limit: a call whose workspace would exceed 64 MiB returns BSFA_ERR_UNSUPPORTED before
 *   anything is enqueued (the keep masks take B * Hq * ceil(N/Bq) * ceil(ceil(Nk/64)/64) * 8
 *   bytes: 8 MiB for one 128K-token sequence with 32 query heads at Bq = 128; FP8 copies do
 *   not fit beyond short sequences). DENSE and RELATIVE take their counter from the array.
 *   Sharing: every call on one device uses that device's one array, which keeps the last
 *   call's contents (each call writes before it reads; nothing needs clearing). Calls that
 *   overlap on one device (another stream, another thread) race on it: the caller orders them.
 * Returns BSFA_OK or an error status as bsfa_prefill does; BSFA_ERR_HIP also when the array's
 * device address cannot be obtained. */
bsfa_status bsfa_prefill_noalloc(const bsfa_problem* p, const void* Q, const void* K,
                                 const void* V, const bsfa_table* table, int32_t budget_slice,
                                 int32_t gate_mode, float log_lambda, void* O,
                                 int32_t* kept_counts, uint64_t* kept_total,
                                 float* debug_block_stat, void* stream);

/* bsfa_prefill over a batch of sequences of different lengths, packed along the token axis
 * (the interface of variable-length attention kernels; "FlashPrefill V2: Block-Sparse Prefill
 * Attention for Long-Context LLM Serving" names varlen scheduling, chunked prefill and
 * continuous batching as what a serving stack needs from a prefill backend). Sequence b owns
 * query tokens [cu_seqlens_q[b], cu_seqlens_q[b+1]) of Q and O and key tokens
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]) of K and V; its Nq_b queries are the last Nq_b of its
 * Nk_b >= Nq_b key positions (a prefix of P_b = Nk_b - Nq_b cached keys, 0 for a whole prefill).
 *   p             batch = number of sequences; seqlen = max_b Nq_b; kv_seqlen = max_b Nk_b (0:
 *                 seqlen); the token and head strides apply, the batch strides are unused
 *   Q, O          device [total_q][Hq][d];  K, V: device [total_k][Hkv][d]
 *   cu_seqlens_q, cu_seqlens_k  device int32 [batch + 1], 4-byte aligned, starting at 0,
 *                 nondecreasing, with Nq_b <= seqlen, Nk_b <= kv_seqlen and Nk_b >= Nq_b (the
 *                 caller guarantees these; they are read on the device only)
 *   kept_counts, debug_block_stat, workspace   as for bsfa_prefill, padded to the longest
 *                 sequence ([batch][Hq][ceil(seqlen/Bq)] ...); entries of query blocks past a
 *                 sequence's end are not written
 *   the rest      as for bsfa_prefill. Under ABSOLUTE each P_b must be a multiple of Bq
 *                 (otherwise the threshold column is floor(P_b/Bq) + i).
 * The results for each sequence are those of bsfa_prefill on that sequence alone. */
bsfa_status bsfa_prefill_varlen(const bsfa_problem* p, const void* Q, const void* K,
                                const void* V, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const bsfa_table* table,
                                int32_t budget_slice, int32_t gate_mode, float log_lambda, void* O,
                                int32_t* kept_counts, uint64_t* kept_total,
                                float* debug_block_stat, void* workspace,
                                uint64_t workspace_bytes, void* stream);

/* bsfa_prefill_varlen with K and V in a paged cache (the layout serving stacks keep their KV
 * cache in; "FlashPrefill V2: Block-Sparse Prefill Attention for Long-Context LLM Serving"
 * names paged KV next to varlen scheduling). Sequence b's key positions 0 .. kv_lens[b] - 1
 * live in pages block_table[b * block_table_stride + 0, 1, ...] of page_size tokens each; its
 * queries are packed in Q / O as for bsfa_prefill_varlen (the last Nq_b of its key positions).
 *   p             as for bsfa_prefill_varlen (kv_seqlen = max_b kv_lens[b]); k_stride[0] and
 *                 v_stride[0] are the page strides, k_stride[1] / [2] the token / head strides
 *   K_pages, V_pages  device [num_pages][page_size][Hkv][d] bf16 (any page order)
 *   cu_seqlens_q  device int32 [batch + 1] query token offsets, 4-byte aligned
 *   kv_lens       device int32 [batch] key tokens per sequence (>= its query tokens)
 *   block_table   device int32 [batch][block_table_stride] page indices, 4-byte aligned;
 *                 block_table_stride >= ceil(kv_seqlen / page_size)
 *   page_size     a positive multiple of 64 tokens (a 64-key tile never straddles two pages;
 *                 BSFA_ERR_SHAPE otherwise)
 *   the rest      as for bsfa_prefill_varlen. The caller guarantees the device-side arrays
 *                 (lengths within the maxima, page indices within K_pages / V_pages).
 * The results equal bsfa_prefill_varlen on the keys gathered from their pages. */
bsfa_status bsfa_prefill_paged(const bsfa_problem* p, const void* Q, const void* K_pages,
                               const void* V_pages, const int32_t* cu_seqlens_q,
                               const int32_t* kv_lens, const int32_t* block_table,
                               int32_t block_table_stride, int32_t page_size,
                               const bsfa_table* table, int32_t budget_slice, int32_t gate_mode,
                               float log_lambda, void* O, int32_t* kept_counts,
                               uint64_t* kept_total, float* debug_block_stat, void* workspace,
                               uint64_t workspace_bytes, void* stream);

/* The absolute gate's keep decisions alone ("Block Sparse Flash Attention", Method: a block
 * is kept when its exact maximum scaled score reaches the threshold T[layer, head, query
 * block]). For every (b, h, i) the exact scores of all off-diagonal blocks j < n_off(i) are
 * computed (no softmax, no V) and bit j % 64 of keep_mask[b][h][i][j / 64] is set iff
 * s_max(i, j) >= T_eff(h, i); the diagonal region is not part of the mask (it is always kept).
 *   p, Q, K, table, budget_slice   as for bsfa_prefill with gate_mode ABSOLUTE (V, O unused)
 *   keep_mask     device uint64 [B][Hq][ceil(N/Bq)][W], W = ceil(ceil(Nk/64)/64), 8-byte
 *                 aligned, one bit per 64-key tile (a kept 128-key block sets both of its
 *                 tiles); every word is written (bits past the off-diagonal tiles are zero)
 *   mask_bytes    size of keep_mask; at least B * Hq * ceil(N/Bq) * W * 8 (mean_correction
 *                 is ignored here). With gate_dtype FP8_E4M3, keep_mask is a 16-byte-aligned
 *                 buffer of at least bsfa_prefill_workspace_bytes(p, ABSOLUTE) bytes (with
 *                 mean_correction 0): the masks, then the FP8 copies this call writes. With
 *                 bf16 scores and mask_bytes >= bsfa_prefill_workspace_bytes(p, ABSOLUTE),
 *                 keep_mask is taken as that workspace and the sweep runs as it does inside
 *                 bsfa_prefill (its workgroups take units from the workspace's counter); the
 *                 masks are the same bit for bit either way
 *   debug_block_stat  as for bsfa_prefill (off-diagonal entries only), or NULL
 *   stream        hipStream_t
 * This is the first of the two launches bsfa_prefill makes when given a workspace; on its own
 * it serves inspection and density monitoring. Same limits and errors as bsfa_prefill
 * (BSFA_ERR_ARG for a NULL or too small keep_mask). */
bsfa_status bsfa_gate_masks(const bsfa_problem* p, const void* Q, const void* K,
                            const bsfa_table* table, int32_t budget_slice, uint64_t* keep_mask,
                            uint64_t mask_bytes, float* debug_block_stat, void* stream);

/* The heavy step of offline threshold calibration ("Block Sparse Flash Attention", Method >
 * Key Designs 1): for every (b, h, i), the maxima of the scaled scores over each visible
 * off-diagonal key block j < n_off(i), and for each budget k their k-th highest value
 * (1-indexed; -INFINITY when n_off(i) < k). Averaging over calibration samples is left to the
 * caller.
 *   p             problem description; V strides, o_stride and out_dtype are ignored
 *   Q, K          as for bsfa_prefill
 *   budgets_host  host int32 [n_budgets], each >= 1
 *   n_budgets     1 .. 16
 *   kth_out       device fp32 [n_budgets][B][Hq][ceil(N/Bq)]
 *   workspace     device, 16-byte aligned, caller-owned scratch of workspace_bytes, or NULL;
 *                 needed only with gate_dtype FP8_E4M3 (at least
 *                 bsfa_calibrate_workspace_bytes(p) bytes): thresholds for an FP8 gate are
 *                 calibrated on its own scores (FP8 copies of Q and K, the FP8 gate sweep's
 *                 block maxima, then the k-th highest); the bf16 scores need none
 *   stream        hipStream_t
 * This library supports seqlen up to 262144 here, whole sequences only (kv_seqlen 0 or equal to
 * seqlen; BSFA_ERR_UNSUPPORTED otherwise). */
bsfa_status bsfa_calibrate_blockmax(const bsfa_problem* p, const void* Q, const void* K,
                                    const int32_t* budgets_host, int32_t n_budgets,
                                    float* kth_out, void* workspace, uint64_t workspace_bytes,
                                    void* stream);

/* Diagnostic: the sustained bf16 matrix-core rate of this device, against which the kernels'
 * executed FLOP rates can be read (the pages quote kernel speed as a share of the matrix peak:
 * "Skipping attention blocks was the easy part", Trusting the numbers). Enqueues one launch of
 * `workgroups` x 4 waves, each issuing 4 * iters v_mfma_f32_32x32x16_bf16 (32768 FLOP each) on
 * register operands, and writes workgroups * 256 floats to `sink` (device, 4-byte aligned).
 * Executed FLOPs = workgroups * 4 * 4 * iters * 32768; the caller times the launch on `stream`.
 * BSFA_ERR_ARG for workgroups < 1, iters < 1 or a NULL sink. */
bsfa_status bsfa_mfma_rate_probe(int32_t workgroups, int32_t iters, float* sink, void* stream);

/* Bytes of workspace bsfa_calibrate_blockmax needs for `p` (0 for bf16 scores): with
 * gate_dtype FP8_E4M3, the masks and FP8 copies of bsfa_prefill_workspace_bytes(p, ABSOLUTE)
 * (without block means and counter), then (on a 256-byte boundary) fp32 [B][Hq][ceil(N/Bq)][ceil(N/Bk)] block
 * maxima. */
uint64_t bsfa_calibrate_workspace_bytes(const bsfa_problem* p);

/* Static description of a status code. Never NULL. */
const char* bsfa_status_string(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* bsfa_last_error(void);

/* ABI version: (major << 16) | minor. Minor 1 adds bsfa_prefill_noalloc; minor 2 ends the
 * absolute gate's workspace with a ticket counter (256 bytes more); minor 3 gives DENSE and
 * RELATIVE a 256-byte workspace (their own ticket counter). Major 3: bsfa_table ends
 * with the budgets array
 * (major 2: bsfa_problem ends with mean_correction and gate_dtype, and
 * bsfa_calibrate_blockmax takes a workspace). */
int32_t bsfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSFA_H_ */
