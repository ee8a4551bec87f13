/*
 * msa.h -- C ABI of libmsa, an MI355X (gfx950) implementation of MiniMax Sparse
 * Attention (MSA) prefill forward and backward.
 *
 * The operator ("feat(minimax-m3): add SM100 MSA sparse attention with custom
 * backward", sections Design and Supported scope) is causal, document-local, top-k
 * block-sparse GQA attention with a fixed topology: 64 query heads, 4 KV heads,
 * 4 index heads, head dim 128, key blocks of 128 tokens and 16 selection slots per
 * (index head, query).  Query head h belongs to index head h / 16, which reads KV
 * head h / 16.  Token t of document d = doc(t) attends to the keys s of the same
 * document with pos(s) <= pos(t) whose block pos(s) / 128 is listed in
 * q2k[h / 16][t][0..15]; -1 marks an unused slot.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless the name ends in _host.  All device arrays
 *     are dense, row-major, 16-byte aligned, on the device that is current when the
 *     call is made.  The caller owns every buffer, including scratch; the library
 *     allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls
 *     only enqueue work on it; none synchronizes the host.
 *   - Return value: MSA_OK (0) or an MSA_ERR_* code.  Argument errors are detected on
 *     the host before anything is enqueued; nothing is written in that case.
 *   - bf16 values are passed as uint16_t bit patterns (msa_bf16).
 *   - Results that use atomics (msa_backward, the CSR column order) are not bitwise
 *     reproducible run to run (pull-request page, Supported scope: atomic
 *     accumulation, not bitwise deterministic).
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed topology (pull-request page, Supported scope). */
#define MSA_NUM_Q_HEADS 64
#define MSA_NUM_KV_HEADS 4
#define MSA_NUM_INDEX_HEADS 4
#define MSA_HEAD_DIM 128
#define MSA_BLOCK 128
#define MSA_TOPK 16
/* Backward task row: 8 queries x 16 heads = 128 rows (msa_backward_sm100 API page,
 * module summary). */
#define MSA_TILE_QUERIES 8
/* Forward work item: up to this many consecutive queries of one document. */
#define MSA_FWD_GROUP 16

typedef uint16_t msa_bf16;

enum {
  MSA_OK = 0,
  MSA_ERR_NULL = 1,      /* a required pointer is NULL */
  MSA_ERR_ALIGN = 2,     /* a device pointer is not 16-byte aligned */
  MSA_ERR_SHAPE = 3,     /* inconsistent sizes or layout */
  MSA_ERR_SCRATCH = 4,   /* a caller buffer is smaller than its *_bytes query */
  MSA_ERR_MODE = 5,      /* unknown dQ accumulation mode */
  MSA_ERR_GRID = 6,      /* grid outside [1, MSA_MAX_GRID] */
  MSA_ERR_LAUNCH = 7,    /* a kernel launch failed */
  MSA_ERR_DEVICE = 8     /* no usable gfx950 device current */
};

/* Bits of the device status word written by msa_build_k2q_csr. */
enum {
  MSA_Q2K_OUT_OF_RANGE = 1, /* an id outside [-1, blk(t)] (ignored) */
  MSA_Q2K_DUPLICATE = 2     /* an id listed twice for one (index head, query) (ignored) */
};

/* How msa_backward forms dQ.  The pages accumulate dQ with 16-bit atomics into a pool
 * (pull-request page, Supported scope; msa_backward_sm100 API page, module summary):
 * modes FP32, BF16X2 and F16X2 do that (fp32 atomics / packed bf16 pair atomics /
 * packed f16 head-pair atomics from the KV-parallel kernel, then a cast).
 * MSA_DQ_RECOMPUTE instead computes dQ in a query-parallel kernel that recomputes P and
 * dS per selected block and stores dQ
 * directly (no pool, no atomics); on gfx950 global atomic throughput, not the matrix
 * cores, bounds the pooled modes.  MSA_DQ_STORED has the KV-parallel kernel, which forms
 * every dS value anyway, store each (query, index head, member slot) dS tile (bf16,
 * 4 KiB) in the scratch, and a query-parallel kernel contract them with K: no
 * recomputation and no atomics, at 4 KiB x 16 x 4 = 256 KiB of scratch per token; the
 * fastest, and the default of the Python binding.  Modes differ in rounding only (dS is
 * rounded to bf16 before its products in all of them). */
enum {
  MSA_DQ_ACCUM_FP32 = 0,
  MSA_DQ_ACCUM_BF16X2 = 1,
  MSA_DQ_RECOMPUTE = 2,
  MSA_DQ_STORED = 3,
  /* Packed-f16 pair atomics into a head-pair-interleaved pool, the pages' default
   * accumulator (pull-request page, Supported scope: FP16 dQ by default;
   * msa_backward_sm100 API page, module summary: head-pair-interleaved pool, packed f16
   * pair reduction).  Pool element (t, h, d) is the f16 at half (h % 2) of 32-bit word
   * (t * 32 + h / 2) * 128 + d; the finalize step de-interleaves it to bf16 dQ. */
  MSA_DQ_ACCUM_F16X2 = 4
};

#define MSA_MAX_GRID 4096

/*
 * Packed-document layout (pull-request page, Design: the layout carries document
 * offsets and token coordinates; every document is padded to a multiple of 128 tokens
 * in the attention K/V workspace).  A host struct holding device arrays:
 *   cu_seqlens [num_docs + 1]: 0 = cu[0] < cu[1] < ... < cu[N] = num_tokens;
 *     document d owns compact tokens [cu[d], cu[d+1]).
 *   cu_ws [num_docs + 1]: cu_ws[d] = sum over e < d of 128 * ceil(L_e / 128), so
 *     document d owns workspace rows [cu_ws[d], cu_ws[d+1]); num_ws_tokens = cu_ws[N].
 * The device arrays must hold what msa_layout_host returns for the same offsets.
 */
typedef struct {
  int32_t num_docs;
  int32_t num_tokens;
  int32_t num_ws_tokens;
  const int32_t *cu_seqlens;
  const int32_t *cu_ws;
} msa_layout;

/* Host: validates cu_seqlens_host [num_docs + 1] (starts at 0, strictly increasing)
 * and writes cu_ws_host [num_docs + 1] and *num_ws_tokens.  MSA_ERR_SHAPE otherwise. */
int msa_layout_host(const int32_t *cu_seqlens_host, int32_t num_docs, int32_t *cu_ws_host,
                    int32_t *num_ws_tokens);

/* ---------------------------------------------------------------------------------
 * Size queries (pure host functions; 0 means the layout is invalid).
 * --------------------------------------------------------------------------------- */
/* Bytes of the CSR scratch (per-row counters). */
size_t msa_csr_scratch_bytes(const msa_layout *layout);
/* Capacity (int32 elements) that `cols` must have: 4 * T * 16. */
size_t msa_csr_cols_capacity(const msa_layout *layout);
/* Bytes of the forward plan buffer. */
size_t msa_plan_bytes(const msa_layout *layout);
/* Bytes of the backward task buffer for a grid of `grid` workgroups. */
size_t msa_tasks_bytes(const msa_layout *layout, int32_t grid);
/* Bytes of the backward scratch (dQ pool of `dq_accum_mode`, if any; fp32 dK/dV pools;
 * MSA_DQ_STORED: the dS tiles, 256 KiB per token). */
size_t msa_bwd_scratch_bytes(const msa_layout *layout, int dq_accum_mode);
/* Grid size msa_build_tasks / msa_backward use by default (one workgroup per CU). */
int32_t msa_default_grid(void);

/* ---------------------------------------------------------------------------------
 * K/V workspace alignment (pull-request page, Design: K/V workspaces with each
 * document padded to a multiple of 128 tokens; msa_backward_sm100 API page,
 * run_backward: W a positive multiple of 128).
 *   K, V: bf16 [T, 4, 128] compact.  Workspace row cu_ws[d] + p holds compact row
 *   cu[d] + p for p < L_d and zeros after; block gb = rows 128 gb .. + 127.  Each of
 *   Kw, Vw, Kt, Vt holds W * 4 * 128 bf16 as [4][W/128] blocks of 16384 (KV head kv,
 *   block gb at element (kv * W/128 + gb) * 16384), in the order the kernels' matrix-
 *   core operands are loaded (each wave-wide 16-byte-per-lane load reads 1 KB of
 *   contiguous memory):
 *   Kw, Vw (row fragments): element (key k, dim d) of a block at
 *     ((k/32 * 8 + d/16) * 64 + (d/8 % 2) * 32 + k%32) * 8 + d%8;
 *   Kt, Vt (transposed fragments): element (key k, dim d) of a block at
 *     ((d/16 * 4 + k/32) * 64 + (k/8 % 4) * 16 + d%16) * 8 + k%8.
 * --------------------------------------------------------------------------------- */
int msa_align_kv(const msa_bf16 *K, const msa_bf16 *V, const msa_layout *layout,
                 msa_bf16 *Kw, msa_bf16 *Vw, msa_bf16 *Kt, msa_bf16 *Vt, void *stream);

/* ---------------------------------------------------------------------------------
 * Indexer block selection: the q2k the operator consumes (pull-request page, Design:
 * the indexer selects a document-local q2k and may align index-K; Supported scope: 4
 * index heads, head dim 128, block 128, top-k 16; Testing: truncated top-16 support).
 * The pages do not state the scoring rule; this library's reading: the score of
 * document-local block b for index head i and the query t at document position p
 * (b <= p / 128) is the largest <IQ[t, i], IK[j, i]> over the keys j of block b with
 * j <= p, accumulated in fp32 from the bf16 inputs.
 *   IQ, IK: bf16 [T, 4, 128] compact (index-Q and index-K projections).
 *   q2k: int32 [4, T, 16] output.  Row (i, t) lists the min(16, p / 128 + 1) blocks of
 *   highest score in ascending id order, ties going to the smaller id, and -1 in the
 *   remaining slots.  Every row of every document is written.
 * Reads IQ and IK only; no scratch.  Argument errors as for every call.
 * --------------------------------------------------------------------------------- */
int msa_index_select(const msa_bf16 *IQ, const msa_bf16 *IK, const msa_layout *layout, int32_t *q2k,
                     void *stream);

/* ---------------------------------------------------------------------------------
 * q2k -> k2q CSR inversion (pull-request page, Design: forward-derived CSR; bindings
 * page: build_k2q_csr).
 *   q2k: int32 [4, T, 16].  Row r = i * NB + gb (NB = W / 128) lists the queries t
 *   whose index head i selects workspace block gb = cu_ws[doc(t)] / 128 + b.
 *   row_ptr: int32 [4 * NB + 1] (exclusive prefix of row lengths).  cols: int32
 *   [msa_csr_cols_capacity]; row r's queries at cols[row_ptr[r] .. row_ptr[r+1]) in
 *   unspecified order.  Slots that are -1, outside [0, blk(t)] or repeat an earlier
 *   slot of the same row are skipped; the latter two set MSA_Q2K_* bits in *status
 *   (device int32, overwritten by this call).
 * --------------------------------------------------------------------------------- */
int msa_build_k2q_csr(const int32_t *q2k, const msa_layout *layout, int32_t *row_ptr,
                      int32_t *cols, int32_t *status, void *scratch, size_t scratch_bytes,
                      void *stream);

/* The same CSR inversion for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no scratch
 * argument; the per-row counters live in a 2 MiB device array of the library (each GPU
 * it runs on holds its own copy until the process ends), cleared by a kernel at the start
 * of every call.  The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Layouts with more than 4 * (2^24 / 128) CSR rows return MSA_ERR_SCRATCH (no
 * layout msa_layout_host accepts has that many).  Calls on one GPU share that array, so
 * calls that overlap on one GPU (other streams, other host threads) race; serialize them.
 * Same arguments, outputs and errors as msa_build_k2q_csr otherwise. */
int msa_build_k2q_csr_noalloc(const int32_t *q2k, const msa_layout *layout, int32_t *row_ptr,
                              int32_t *cols, int32_t *status, void *stream);

/* ---------------------------------------------------------------------------------
 * Forward plan (the forward schedule; bindings page: fmha_sm100_plan).  Cuts every
 * document into groups of MSA_FWD_GROUP consecutive queries; each (index head, group)
 * is one work item.  Items of one head are ordered by cost (member slots) descending,
 * ties in document order, and heads are interleaved: item p belongs to head p % 4.
 * Each item carries its walk list: the member blocks of its queries in ascending order,
 * each with the bit mask of the item's queries (bit u = query t0 + u) that select it;
 * msa_forward and the dQ step of msa_backward walk these lists.
 * Layout of `plan` (int32 words; NI = 4 * (ceil(T / MSA_FWD_GROUP) + num_docs)):
 *   [0] item count; items {i, t0, n, doc} at [16 + 4p];
 *   list lengths at [16 + 4 NI + p]; list of item p at
 *   [16 + 4 NI + round_up(NI, 4) + 2 * 256 * p + 2e] = {block, mask}, e < length.
 * q2k as above.
 * --------------------------------------------------------------------------------- */
int msa_plan(const msa_layout *layout, const int32_t *q2k, void *plan, size_t plan_bytes,
             void *stream);

/* ---------------------------------------------------------------------------------
 * Forward (pull-request page, Design: Q[T,64,128], K/V, q2k -> O[T,64,128] + LSE).
 *   Q: bf16 [T, 64, 128].  Kw and Vt from msa_align_kv.  plan from msa_plan (its walk
 *   lists carry the selection).  scale: the softmax scale applied to Q K^T, finite and
 *   > 0 (else MSA_ERR_SHAPE).
 *   O: bf16 [T, 64, 128].  LSE: fp32 [T, 64], natural log of the sum of exp(scores),
 *   scores including `scale`; -inf (and O = 0) for a row with no keys.
 * --------------------------------------------------------------------------------- */
int msa_forward(const msa_bf16 *Q, const msa_bf16 *Kw, const msa_bf16 *Vt, const msa_layout *layout,
                const void *plan, float scale, msa_bf16 *O, float *LSE, void *stream);

/* ---------------------------------------------------------------------------------
 * Backward preprocessing (pull-request page, Custom kernel: delta preprocessing).
 *   delta[t, h] = sum_c dO[t,h,c] * O[t,h,c] in fp32 from the bf16 O and dO [T,64,128].
 * --------------------------------------------------------------------------------- */
int msa_backward_preprocess(const msa_bf16 *O, const msa_bf16 *dO, int32_t num_tokens,
                            float *delta, void *stream);

/* ---------------------------------------------------------------------------------
 * Backward task tables + CTA walk (pull-request page, Changelog / Custom kernel: task
 * construction from the saved forward schedule with exact counts and device-side CTA
 * scheduling; msa_backward_sm100 API page: 128-row tiles of 8 queries x 16 heads
 * bucketed by (index head, key block)).  From the CSR: bucket r holds
 * ceil(len_r / 8) task rows, every one full except the last.  Layout of `tasks`
 * (int32 words):
 *   [0] R (total rows), [1..4] rows per index head, [5..8] first row of each head,
 *   [9] grid, [10] row capacity Rmax;
 *   cta bounds at [64 ...]: (4 * (grid + 1)) words, workgroup c walks rows
 *     [cta[i*(grid+1)+c], cta[i*(grid+1)+c+1]) of index head i, = first_i +
 *     floor(c * rows_i / grid);
 *   meta at word msa_tasks_meta_offset(): Rmax x {r, n_valid, flags, k} (flags bit0 =
 *     first row of its bucket, bit1 = last);
 *   qrows, qpos, qtile: Rmax x 8 int32 each (query ids; document-local positions;
 *     stored-dS tile index (t * 4 + i) * 16 + j with j the first slot of q2k[i][t]
 *     listing the bucket's block; -1 pad).  q2k must be the device q2k the CSR was built
 *     from (the same array contents; a different q2k gives wrong tile indices, unchecked).
 * Rows inside one bucket appear in ascending k; their query sets follow the CSR order.
 * --------------------------------------------------------------------------------- */
size_t msa_tasks_meta_offset(int32_t grid);
int msa_build_tasks(const msa_layout *layout, const int32_t *row_ptr, const int32_t *cols,
                    const int32_t *q2k, int32_t grid, void *tasks, size_t tasks_bytes, void *stream);

/* ---------------------------------------------------------------------------------
 * Backward (msa_backward_sm100 API page, run_backward and module summary):
 *   Q, dO: bf16 [T, 64, 128]; Kw, Vw, Kt from msa_align_kv; LSE fp32 [T, 64] from
 *   msa_forward; delta from msa_backward_preprocess; q2k and plan those the CSR and
 *   the forward were built from (the stored-dS and recompute modes look blocks up in
 *   them; a different q2k is not detected and gives wrong dQ); tasks from
 *   msa_build_tasks and `grid` the value it was built with (the
 *   KV-parallel launch uses that many workgroups).  scale: the forward's softmax scale
 *   (finite and > 0, else MSA_ERR_SHAPE).  Writes dQ bf16 [T, 64, 128] and
 *   dK, dV bf16 [T, 4, 128] in compact token order.  scratch >=
 *   msa_bwd_scratch_bytes(layout, dq_accum_mode): the dQ pool of the pooled modes and
 *   fp32 dK/dV pools, zeroed by this call, then (MSA_DQ_STORED) the dS tiles, 4 KiB per
 *   (token, index head, q2k slot), written before they are read (not zeroed).  The
 *   scratch holds no state between calls.  Calls that share a scratch buffer must not
 *   overlap.
 * --------------------------------------------------------------------------------- */
int msa_backward(const msa_bf16 *Q, const msa_bf16 *Kw, const msa_bf16 *Vw, const msa_bf16 *Kt,
                 const msa_bf16 *dO, const float *LSE, const float *delta, const int32_t *q2k,
                 const void *plan, const void *tasks, int32_t grid, const msa_layout *layout,
                 float scale, int dq_accum_mode, msa_bf16 *dQ, msa_bf16 *dK, msa_bf16 *dV,
                 void *scratch, size_t scratch_bytes, void *stream);

/* Timing hook.  `events` holds MSA_TIMING_EVENTS hipEvent_t handles (or is NULL, which
 * turns the hook off).  While set, calls from this host thread record, on the call's
 * stream: events[0] / [1] right before / after the forward kernel launches of
 * msa_forward; events[2] / [3] around the KV-parallel backward kernel of msa_backward
 * (dK/dV, plus the dQ atomics of the pooled modes); events[4] / [5] around its
 * query-parallel dQ kernel (MSA_DQ_RECOMPUTE and MSA_DQ_STORED).  The array is copied; the caller keeps the events alive while
 * the hook is set.  Lets a caller time each kernel alone. */
#define MSA_TIMING_EVENTS 6
void msa_set_timing_events(void *const *events);

/* Short description of a return code. */
const char *msa_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
