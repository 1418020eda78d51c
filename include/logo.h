/*
 * logo.h — C ABI of the token-level dynamic local-global attention forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (pages: "LoGo: Token-Level Dynamic Local-Global Attention",
 * abstract; "Learning When to Attend", section "The Architecture of
 * Conditional Attention"; "Local-global attention", attention-mask sketch):
 *
 *   every query i attends causally over its last W keys
 *       L(i) = [max(0, i-W+1), i]                          (local branch)
 *   a gate logit per (batch, token) and a budget controller pick, per
 *   sequence, the k = ceil(rho*n) tokens with the largest logits, ties to
 *   the lower position                                     (selection S)
 *   the tokens in S also attend over the whole causal prefix
 *       G(i) = [0, i]                                      (global branch)
 *   o_i = o_local_i + sigmoid(gate_i) * o_global_i   for i in S
 *   o_i = o_local_i                                   otherwise
 *
 * Scores are scale * <q_i, k_j>; the softmax is exact (no approximation of
 * either branch). Grouped-query heads: query head h reads key/value head
 * h / (Hq/Hkv).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers: device pointers (hipMalloc'ed or equivalent), 16-byte aligned,
 *   owned by the caller. The library never allocates, frees or keeps device
 *   memory. Scratch space comes from the caller's workspace argument.
 * Layouts (row-major; the d elements of one row are always contiguous):
 *   q, o          [B][Hq][n][d]     dtype = problem.dtype
 *   k, v          [B][Hkv][n][d]    dtype = problem.dtype
 *     q, k, v and o may instead be strided views: problem.q_strides etc.
 *     give the (batch, head, token) strides in elements (see logo_problem);
 *     all three zero means the contiguous layout above.
 *   gate          [B][n]            float32 logits
 *   mask          [B][n]            uint8, 1 = selected
 *   idx           [B][k]            int32, selected positions, ascending
 *   rank          [B][n]            int32, index of the token in idx or -1
 *   o_local       [B][Hq][n][d]     float32
 *   o_global      [B][Hq][k][d]     float32, rows in idx order
 * Streams: `stream` is a hipStream_t (NULL = the default stream). Every call
 *   only enqueues work on it and returns; nothing synchronises.
 * Errors: argument errors are detected on the host before anything is
 *   enqueued; outputs are then untouched. A failed kernel launch returns
 *   LOGO_ERR_HIP. logo_last_error() gives a readable message for the last
 *   failure on the calling thread. No C++ exception crosses this boundary.
 * Empty problems (B == 0 or n == 0) are valid and enqueue nothing.
 * Supported: d in {64, 128}; dtype LOGO_F32 or LOGO_BF16 (float32
 *   accumulation in both); 1 <= window; 0 <= rho <= 1; Hq % Hkv == 0;
 *   n < 2^30; B*Hq*n*d < 2^62; for strided views, ((n-1)*token stride + d)
 *   times the element size below 2^31 bytes.
 */
#ifndef LOGO_H
#define LOGO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LOGO_OK = 0,
  LOGO_ERR_INVALID_ARG = 1,  /* NULL/misaligned pointer, bad size or ratio */
  LOGO_ERR_UNSUPPORTED = 2,  /* well-formed but not built (e.g. d = 96)    */
  LOGO_ERR_WORKSPACE = 3,    /* workspace missing or smaller than needed  */
  LOGO_ERR_HIP = 4           /* a HIP runtime call or launch failed       */
} logo_status;

typedef enum { LOGO_F32 = 0, LOGO_BF16 = 1 } logo_dtype;

/* One attention layer's problem description. */
typedef struct {
  int64_t B;       /* batch (sequences)                                     */
  int64_t Hq;      /* query heads                                           */
  int64_t Hkv;     /* key/value heads; Hq % Hkv == 0                        */
  int64_t n;       /* tokens per sequence                                   */
  int64_t d;       /* head dimension: 64 or 128                             */
  int64_t window;  /* W >= 1: keys each query reads locally, itself included */
  double rho;      /* target global ratio in [0, 1]; k = ceil(rho * n)      */
  float scale;     /* score scale; 0 means 1/sqrt(d)                        */
  int32_t dtype;   /* logo_dtype of q, k, v, o                              */
  /* Strides in elements of q, k, v and o along (batch, head, token); the d
   * stride is 1. {0, 0, 0} selects the contiguous [B][H][n][d] layout. A
   * set stride triple must have every stride >= 0, a token stride >= d,
   * and every stride times the element size a multiple of 16 bytes. Inputs
   * may overlap (a batch or head stride of 0 broadcasts); o must not: its
   * strides, sorted, must each be at least the previous stride times that
   * dimension's extent (LOGO_ERR_INVALID_ARG otherwise). The intermediate
   * o_local / o_global / workspace buffers are always contiguous. */
  int64_t q_strides[3];
  int64_t k_strides[3];
  int64_t v_strides[3];
  int64_t o_strides[3];
} logo_problem;

/* Number of selected tokens per sequence: ceil(rho * n) computed in double
 * and clamped to [0, n] (LoGo abstract: the budget controller keeps a target
 * global ratio). Returns -1 when rho is NaN or n < 0. */
int64_t logo_target_count(double rho, int64_t n);

/* Bytes of workspace logo_forward needs for this problem (float32 local
 * outputs of the selected rows: B*Hq*k*d*4, rounded up to 256, then one
 * int32 per (b, kv head) for the global branch's work queues, rounded up to
 * 256). A bf16 problem whose global branch has fewer than 512 workgroups
 * (one per 32 selected rows of up to 4 query heads of a kv head:
 * B*Hkv*ceil(ceil(k/32)*Hq/Hkv / 4)) splits each workgroup's keys into
 * s = min(8, ceil(512 / workgroups), floor(ceil(n/64) / 4)) ranges when
 * that is 2 or more, and then adds s*B*Hq*k*(d+4)*4 bytes of float32
 * partials, rounded up to 256. A bf16 problem with k > 0 that does not
 * split and whose B*Hkv is a multiple or a divisor of 8 runs the single
 * launch (see logo_forward) and adds B*(n-k)*4 bytes (the unselected
 * positions), rounded up to 256. Writes 0 when nothing is needed. Errors:
 * LOGO_ERR_INVALID_ARG / _UNSUPPORTED as for logo_forward. */
logo_status logo_workspace_size(const logo_problem* p, size_t* bytes);

/* Budget controller + compaction (LoGo abstract: threshold-based budget
 * controller; "Learning When to Attend": one binary decision per token).
 * For each sequence b, selects the k = ceil(rho*n) largest gate[b][.]
 * (ties to the lower position, -0.0 == +0.0, NaN below every number) and
 * writes mask, idx (ascending) and rank. The result is unique and
 * bit-exact. idx may be NULL when k == 0. */
logo_status logo_select_queries(const logo_problem* p, const float* gate,
                                uint8_t* mask, int32_t* idx, int32_t* rank,
                                void* stream);

/* Local branch for every query: softmax over L(i) = [max(0,i-W+1), i],
 * times V ("Local-global attention", attention-mask sketch: causal and
 * within-window). Writes o_local [B][Hq][n][d] float32. */
logo_status logo_local_attn(const logo_problem* p, const void* q, const void* k,
                            const void* v, float* o_local, void* stream);

/* Global branch for the selected queries only: softmax over G(i) = [0, i],
 * times V ("Learning When to Attend": exact attention over the full context
 * for a sparse subset of query tokens). idx [B][k] are the rows (ascending
 * positions, each in [0, n)); writes o_global [B][Hq][k][d] float32 in idx
 * order. Nothing is enqueued when k == 0 (idx, o_global may be NULL). */
logo_status logo_global_attn_sparse(const logo_problem* p, const void* q,
                                    const void* k, const void* v,
                                    const int32_t* idx, float* o_global,
                                    void* stream);

/* Gated combine: o = o_local + sigmoid(gate) * o_global[rank] where
 * rank >= 0, o = o_local elsewhere; float32 arithmetic, one rounding to the
 * output dtype. o_global may be NULL when k == 0. */
logo_status logo_combine(const logo_problem* p, const float* o_local,
                         const float* o_global, const int32_t* rank,
                         const float* gate, void* o, void* stream);

/* The whole layer in one call: selection, local branch, global branch on S,
 * combine, on one stream with no host synchronisation. Writes o and the
 * selection (mask, idx, rank). `workspace` must hold logo_workspace_size
 * bytes (may be NULL when that is 0). Output equals logo_select_queries ->
 * logo_local_attn -> logo_global_attn_sparse -> logo_combine up to float32
 * rounding order. Two bf16 forms take another order and then agree with
 * those calls to the bf16 parity tolerance rather than bit for bit: a
 * global branch split into key ranges (see logo_workspace_size), where each
 * range rounds its probabilities to bf16 against its own running maximum
 * (such a problem runs the split global branch and the local branch in one
 * launch, then merges the ranges); and the single launch (see logo_workspace_size for when it applies),
 * where one kernel does every row: a selected row walks its causal prefix
 * once, from the diagonal down, its window's keys first, so the running
 * state after the window is its local output and at the end its global
 * output, and the unselected rows do the local branch alone. */
logo_status logo_forward(const logo_problem* p, const void* q, const void* k,
                         const void* v, const float* gate, void* o,
                         uint8_t* mask, int32_t* idx, int32_t* rank,
                         void* workspace, size_t workspace_bytes, void* stream);

/* The forward for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation. Same arguments, results and errors as logo_forward, without
 * the workspace: its scratch is one array of LOGO_NOALLOC_SCRATCH_BYTES in
 * the library's device code, which every GPU the library runs on holds
 * from the library's first use there until the process ends. No call
 * allocates or frees memory. Returns LOGO_ERR_WORKSPACE, before enqueueing
 * anything, when logo_workspace_size exceeds LOGO_NOALLOC_SCRATCH_BYTES
 * (the headline 32K layer needs about 107 MB; the 128K one does not fit).
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents: calls that overlap on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller. */
#define LOGO_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
logo_status logo_forward_noalloc(const logo_problem* p, const void* q,
                                 const void* k, const void* v,
                                 const float* gate, void* o, uint8_t* mask,
                                 int32_t* idx, int32_t* rank, void* stream);

/* ---- training: forward that saves statistics, and the backward --------
 *
 * The gate is learned (LoGo abstract) and the method is trained ("Learning
 * When to Attend", section "Empirical Validation and System Optimization"),
 * but no page prints a backward pass; the one here is the chain rule of the
 * forward above with the selection S held fixed: choosing the top-k logits
 * has no derivative and the pages give no rule for passing a gradient
 * through it, so the gate gets gradient only through sigmoid(gate_i) on
 * selected tokens, summed over the query heads that share it:
 *   dgate_i = g_i (1 - g_i) sum_h <dout_{h,i}, o_global_{h,i}>   (i in S)
 *   dgate_i = 0                                                  otherwise
 * and q, k, v get the softmax-attention gradients of both branches (the
 * global one with upstream gradient g_i dout_i); a kv head sums over its
 * query heads. */

/* As logo_forward (same o, mask, idx, rank), and also writes what
 * logo_backward needs:
 *   lse_local   [B][Hq][n]    float32: log sum_j exp(scale <q_i, k_j>) over
 *                             L(i) (natural log) for every row
 *   lse_global  [B][Hq][k]    float32: the same over G(i), rows in idx order
 *   o_local_sel [B][Hq][k][d] float32: local output of the selected rows
 *                             (this buffer is also the forward's workspace)
 *   o_global    [B][Hq][k][d] float32: global output of the selected rows
 * The four may be NULL only in the cases noted (k == 0: all but lse_local).
 * Errors: as logo_forward. */
logo_status logo_forward_train(const logo_problem* p, const void* q, const void* k,
                               const void* v, const float* gate, void* o,
                               uint8_t* mask, int32_t* idx, int32_t* rank,
                               float* lse_local, float* lse_global,
                               float* o_local_sel, float* o_global, void* stream);

/* Bytes of workspace logo_backward needs (row terms and the selected rows'
 * queries and gated upstream gradients, gathered: about
 * 2*B*Hq*(n + k)*4 + 2*B*Hq*k*d*sizeof(dtype)). */
logo_status logo_backward_workspace_size(const logo_problem* p, size_t* bytes);

/* Gradients of the layer for upstream gradient `dout` (o's dtype and
 * layout, o_strides). Inputs: q, k, v, gate and the outputs of
 * logo_forward_train for them (o, idx, rank, lse_local, lse_global,
 * o_local_sel, o_global). Outputs, float32, contiguous, fully overwritten:
 *   dq [B][Hq][n][d], dk and dv [B][Hkv][n][d], dgate [B][n].
 * No atomics: results are bitwise reproducible run to run.
 * Errors: as logo_forward; LOGO_ERR_WORKSPACE if the workspace is missing
 * or smaller than logo_backward_workspace_size. */
logo_status logo_backward(const logo_problem* p, const void* q, const void* k,
                          const void* v, const float* gate, const void* o,
                          const void* dout, const int32_t* idx, const int32_t* rank,
                          const float* lse_local, const float* lse_global,
                          const float* o_local_sel, const float* o_global,
                          float* dq, float* dk, float* dv, float* dgate,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- routed forward: the gate computed from the local branch ----------
 *
 * "Learning When to Attend" (section "The Architecture of Conditional
 * Attention") runs local attention for every token first and then routes
 * each token; LoGo (abstract) learns the gate. Here the router is a linear
 * map of the token's local output over all query heads (the pages give no
 * router architecture; the plainest reading):
 *   gate[b][i] = router_bias + sum_h <router_w[h], o_local[b][h][i]>
 * then, as in logo_forward, the top-k selection on those logits, the global
 * branch for the selected rows and o = o_local + sigmoid(gate) o_global.
 * Order of work: local -> router -> select -> global, one stream.
 *   router_w   [Hq][d] float32 (device)
 *   gate       [B][n]  float32 output: the computed logits (the selection and
 *              the combine use exactly these values)
 *   o, mask, idx, rank as logo_forward.
 * Workspace: logo_routed_workspace_size bytes (the float32 local output of
 * every row, B*Hq*n*d*4, B*Hq*n*4 of per-head partial logits and B*Hkv*4
 * of work queues, each rounded up to 256).
 * Errors: as logo_forward; LOGO_ERR_INVALID_ARG for a non-finite bias. */
logo_status logo_routed_workspace_size(const logo_problem* p, size_t* bytes);
logo_status logo_forward_routed(const logo_problem* p, const void* q, const void* k,
                                const void* v, const float* router_w, float router_bias,
                                float* gate, void* o, uint8_t* mask, int32_t* idx,
                                int32_t* rank, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---- threshold budget controller and the decode step ------------------
 *
 * LoGo (abstract) holds the target global ratio with a threshold-based
 * budget controller; "Learning When to Attend" (section "Empirical
 * Validation and System Optimization") reads the full context at decode
 * time only for tokens routed to it. Readings (the pages give no formulas):
 * a token is selected iff gate > tau (NaN never); the running controller
 * moves tau by eta (selected - rho) after each decision, a quantile tracker
 * whose selected fraction settles at rho using only past tokens. */

/* Calibrated threshold from a prefill's exact top-k selection: tau[b] is the
 * largest gate[b][i] with mask[b][i] == 0 (NaN excluded), -inf when every
 * token was selected, so "gate > tau" reproduces the selection on distinct
 * logits. gate, mask [B][n]; tau [B] float32 out. n >= 1. */
logo_status logo_calibrate_threshold(const logo_problem* p, const float* gate,
                                     const uint8_t* mask, float* tau, void* stream);

/* Threshold selection of whole sequences: mask[b][i] = gate[b][i] > tau[b];
 * idx [B][n] int32 gets the selected positions ascending, then -1;
 * count [B] int32 the number selected. (The budget is not enforced: the
 * count follows the logits.) */
logo_status logo_select_threshold(const logo_problem* p, const float* gate,
                                  const float* tau, uint8_t* mask, int32_t* idx,
                                  int32_t* count, void* stream);

/* One decode step per sequence. */
typedef struct {
  int64_t B;       /* sequences                                              */
  int64_t Hq;      /* query heads; G = Hq / Hkv in 1..16 for bf16 caches of
                      at most 1023 sequences, else G in {1, 2, 4, 7, 8}       */
  int64_t Hkv;     /* key/value heads                                        */
  int64_t cap;     /* cache capacity (positions per sequence and kv head)    */
  int64_t d;       /* head dimension: 64 or 128                              */
  int64_t window;  /* W >= 1                                                 */
  double rho;      /* target global ratio in [0, 1]                          */
  float eta;       /* controller step >= 0 (0 freezes tau)                   */
  float scale;     /* score scale; 0 means 1/sqrt(d)                         */
  int32_t dtype;   /* logo_dtype of q, caches and o                          */
} logo_decode_problem;

/* Bytes of workspace logo_decode_step needs (per-chunk partial softmax
 * states: B*Hq*ceil(cap/1024)*2*(d+4)*4). */
logo_status logo_decode_workspace_size(const logo_decode_problem* p, size_t* bytes);

/* The newest token of each sequence attends over its cache:
 *   q        [B][Hq][d]           dtype
 *   k_cache, v_cache [B][Hkv][cap][d] dtype, contiguous; positions
 *            0 .. lens[b]-1 valid, the newest token's own key/value included
 *   lens     [B] int32 in [1, cap] (values outside are clamped into it)
 *   gate     [B] float32 logit of the newest token
 *   tau      [B] float32 threshold, read then updated in place:
 *            selected[b] = gate[b] > tau[b]; tau[b] += eta (selected[b] - rho)
 *   o        [B][Hq][d] dtype: o_local over the last W cached keys, plus
 *            sigmoid(gate) o_global over the whole cache when selected
 *   selected [B] uint8 out.
 * Reads each needed cached key and value once (the kv head's query heads
 * share it); unselected sequences read only their window. Errors:
 * LOGO_ERR_INVALID_ARG (bad sizes, ratio, step, scale or dtype, NULL or
 * misaligned pointers), LOGO_ERR_UNSUPPORTED (head dimension, group size,
 * sizes past the 32-bit work counts), LOGO_ERR_WORKSPACE, LOGO_ERR_HIP;
 * nothing is enqueued on an argument error. */
logo_status logo_decode_step(const logo_decode_problem* p, const void* q,
                             const void* k_cache, const void* v_cache,
                             const int32_t* lens, const float* gate, float* tau,
                             void* o, uint8_t* selected, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---- packed variable-length batches --------------------------------------
 *
 * Several examples packed into one token stream ("Local-global attention",
 * implementation-sketch notes: packing needs per-example boundaries so no
 * token attends across them). The problem has B = 1 and n = T, the total
 * number of tokens; cu_seqlens [E+1] (ascending, cu[0] = 0, cu[E] = T)
 * splits the stream into examples. Every example is its own sequence: the
 * local window and the global prefix stop at its first token, and its
 * budget is k_e = ceil(rho * n_e) of its own gate logits (ties to the lower
 * position). q, o [1][Hq][T][d] and k, v [1][Hkv][T][d] with the problem's
 * strides (a token-major [T][H][d] layout is a strided view); gate, mask,
 * rank [T]; idx [K] with K = logo_varlen_selected_count: the examples'
 * selections concatenated, absolute token positions (ascending); rank is a
 * token's index in idx or -1. Inconsistent cu_seqlens on the device (not
 * what logo_varlen_selected_count was given) give undefined results but no
 * access outside the buffers: idx writes past K are dropped. */

/* K = sum over examples of ceil(rho * (cu[e+1] - cu[e])), from a host copy of
 * cu_seqlens; -1 for a bad ratio, cu[0] != 0 or decreasing offsets. */
int64_t logo_varlen_selected_count(double rho, const int32_t* cu_seqlens_host,
                                   int64_t n_examples);

/* Workspace of logo_forward_varlen: 16 B per example, 4 B per token, the
 * float32 local outputs of the selected rows (Hq*K*d*4), the bf16 work
 * order, and, where the single launch runs the stream, 4 B per unselected
 * token; each part 256-aligned. */
logo_status logo_varlen_workspace_size(const logo_problem* p, int64_t n_examples,
                                       int64_t total_selected, size_t* bytes);

/* The forward over a packed batch (cu_seqlens is a device pointer). Where
 * logo_forward would take its single launch for a stream of this size
 * (bf16, d in {64, 128}, K > 0, no key-range split, Hkv a multiple or a
 * divisor of 8), so does this call: the selection also lists the unselected
 * tokens, and one launch computes every row, the selected ones walking their
 * example's prefix once for both branches (results then agree with the two
 * launches to the parity tolerance, not bit for bit). */
logo_status logo_forward_varlen(const logo_problem* p, const int32_t* cu_seqlens,
                                int64_t n_examples, int64_t total_selected,
                                const void* q, const void* k, const void* v,
                                const float* gate, void* o, uint8_t* mask,
                                int32_t* idx, int32_t* rank, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* logo_status_string(logo_status s);

/* Message describing the last failure on the calling thread ("" if none). */
const char* logo_last_error(void);

/* Kernel timing for measurement. Between logo_profile_begin() and
 * logo_profile_end(), logo_forward records a HIP event pair around each of
 * its kernels on the caller's stream (at most 4096 pairs; later launches go
 * unrecorded); so do logo_forward_train, logo_backward,
 * logo_forward_routed and logo_decode_step. logo_profile_end() waits for those events and writes,
 * per stage (0 select, 1 local, 2 global, 3 combine, 4 backward row terms and
 * dgate, 5 backward dk/dv, 6 backward dq, 7 router logits, 8 decode: chunk
 * partials and their reduction, 9 both attention branches in one launch,
 * 10 the local band and the key-range-split global branch in one launch
 * plus their merge),
 * the summed milliseconds
 * and the number of launches into arrays of `n_stages` entries. The events
 * are timing-only (created without the system-scope fence, so recording one
 * flushes no cache); they order nothing for the caller. */
logo_status logo_profile_begin(void);
logo_status logo_profile_end(double* stage_ms, int64_t* stage_launches,
                             int32_t n_stages);

#ifdef __cplusplus
}
#endif

#endif /* LOGO_H */
