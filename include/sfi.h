/*
 * sfi.h -- C ABI of libsfi: slow-fast decode attention (SFI) and
 * verification-guided sparse selection (Vegas) on AMD Instinct MI355X (gfx950).
 *
 * Sources:
 *   [SFI]   "Slow-Fast Inference: Training-Free Inference Acceleration via
 *           Within-Sentence Support Stability" (gist.science/it|pt|ko/paper/
 *           2603.12038): technical summary, section 1 (every decode step
 *           attends the whole cached history), section 3.A / 2.A (fast steps
 *           over sinks + recent window + selected memory; slow steps with
 *           dense attention at boundaries or when the reuse budget is spent),
 *           section 3.B / 2.B (selector: evidence from the slow step's
 *           attention, prior from key norms and positions, closed-form
 *           reverse-KL fusion s = (1-lam) f + lam r, Top-K).
 *   [Vegas] "Vegas: Decodifica Auto-Speculativa con Attenzione Sparsa Guidata
 *           dalla Verifica" (gist.science/it/paper/2602.07223): section 2
 *           (verify with full attention, select from its logits, draft with
 *           sparse attention), section 2.A (argmax over |T| = k of the
 *           logits summed over the verified queries and all query heads),
 *           section 2.B (Collect-2-Query), section 3 (pre-softmax logits).
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns all
 *     memory, including the workspace `ws` (size from the matching
 *     *_workspace_bytes call).  No call allocates, frees or synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream) and the call returns.  Argument errors are reported
 *     synchronously, before anything is enqueued.  SFI_ERR_HIP means a launch
 *     was rejected; faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - K/V/Q are bf16 bit patterns (uint16_t).  Outputs are fp32.  Logits are
 *     q.k / sqrt(d); query head h reads kv head h / (Hq / Hkv).
 *   - K, V, queries, attention outputs and compact copies are 16-byte
 *     aligned and workspaces 256-byte aligned (SFI_ERR_RANGE otherwise);
 *     device allocators return such addresses.
 *   - A batch is a list of sequence ids (`batch_ids`, int32, device, length
 *     `batch_n`; NULL means 0..batch_n-1).  Results are written at each
 *     sequence's own slot b, so full-batch buffers can be shared by calls
 *     that touch disjoint subsets.  Ids must be distinct and < B.
 *   - Calls on one stream run in order; calls that share a workspace must be
 *     ordered by the caller.  Results are bitwise repeatable (no floating-
 *     point atomics; reductions run in a fixed order).
 */
#ifndef SFI_H
#define SFI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SFI_OK = 0,
  SFI_ERR_NULL = -1,        /* a required pointer is NULL */
  SFI_ERR_SHAPE = -2,       /* inconsistent or unsupported sizes */
  SFI_ERR_RANGE = -3,       /* a parameter outside its documented range */
  SFI_ERR_WORKSPACE = -4,   /* ws_bytes smaller than required */
  SFI_ERR_UNSUPPORTED = -5, /* valid request this build has no kernel for */
  SFI_ERR_HIP = -6          /* the HIP runtime rejected a launch */
} sfi_status;

/* The KV cache of one attention layer.
 *   Contiguous (page_table == NULL): k, v are [B][Hkv][cap][d].
 *   Paged: k, v are a pool [num_pages][Hkv][page_size][d]; logical row j of
 *   sequence b lives in page page_table[b * max_pages + j / page_size] at
 *   offset j % page_size.  max_seq_len <= 4,194,304 for a paged cache (else
 *   SFI_ERR_UNSUPPORTED).
 * seq_len[b] (device) is the number of cached keys of sequence b, including
 * the token(s) being decoded.  max_seq_len [host] bounds seq_len over every
 * sequence a call touches; it sizes grids and workspaces.  Device values are
 * trusted only within bounds: seq_len is clamped to [0, max_seq_len], page ids
 * to [0, num_pages), and listed sequence ids outside [0, B) are skipped, so a
 * corrupt argument yields wrong numbers, never an out-of-bounds access.
 * Layout note: a contiguous cache whose (sequence, kv head) stride, cap * d
 * * 2 bytes, sits on certain power-of-two sums aliases in the HBM channel
 * mapping (2^23 + 2^16 bytes made fast steps 2x slower on MI355X); padding
 * cap by a few dozen rows avoids it.
 *
 * Fused append [SFI technical summary, section 1: the cache grows by each
 * decode step's own key and value]: k_new, v_new ([B][Hkv][d] bf16 bits,
 * 16-byte aligned; both NULL or both set) hold that row of every sequence.
 * Set, the step calls (sfi_slow_step, sfi_fast_step, sfi_fast_step_noalloc,
 * sfi_fast_step_compact, sfi_decode_step, sfi_decode_step_select,
 * sfi_decode_layer_step) take cache row seq_len[b] - 1 of each listed
 * sequence from them and store it into the cache (k, v must then be
 * writable): the same results as sfi_append_kv with T = 1 followed by the
 * step, without the extra launch.  Sequences a call does not list are not
 * appended.  sfi_append_kv, sfi_verify_* and sfi_slow_step_window return
 * SFI_ERR_RANGE when they are set; sfi_compact_selected ignores them.
 *
 * Key-norm statistics [SFI technical summary, section 3.B: the prior
 * standardises each key's norm by the mean and spread of the row's key
 * norms]: norm_stats ([B][Hkv][2] fp64, 8-byte aligned, device) holds for
 * every (sequence b, kv head g) the sum and the sum of squares of the
 * L2 norms of the cache rows written so far (rows j < seq_len[b], less a
 * row that a fused append is about to write).  Set, the calls keep it
 * current: step calls add the norm of each fused-append row, sfi_append_kv
 * adds its rows' norms, and the calls that form the selector's prior
 * (sfi_decode_step_select, sfi_decode_layer_step) overwrite the sums of
 * their slow sequences with the exact sums of their pass (their fused rows
 * included).  Rows written by other means leave it stale.  With
 * norm_stats_valid = 1 as well, the caller vouches that the sums are
 * current for every slow sequence of the call, and sfi_decode_step_select
 * then forms the prior from them: its attention pass computes the prior
 * weights and its finalize runs the selection's key pass, one launch fewer
 * (Soft-NMS and exclusivity keep the separate passes).  The norms are fp32
 * roundings summed in fp64, so the prior matches the one formed from the
 * pass up to rounding (near-tie keys may select differently).
 *
 * Row-count hints (launch planning only; they change no step of the
 * method, and serve batches whose sequences differ much in length):
 * slow_len_host and fast_len_host are host arrays in the order of the
 * call's slow list and fast list (the one list of sfi_slow_step and
 * sfi_fast_step), read during the call only.  slow_len_host[z] is the
 * seq_len of the z-th slow entry (0..max_seq_len); fast_len_host[z] bounds
 * the rows of the z-th fast entry's row list, at least
 * min(seq_len, n_sink + window) plus the entry's largest sel_count
 * (0..n_sink + window + sel_k).  Set, the split plan is sized from the
 * longest hint instead of max_seq_len, and where the entries' counts
 * differ (a tenth or more of such a plan's workgroups would find no rows)
 * it gives each listed entry only the workgroups its own rows need (a work
 * table of at most 256 entries; longer lists keep the plain plan).  A hint
 * outside its range is SFI_ERR_RANGE; one below the true count leaves the
 * rows past it out of the result, and the fused append of a row past it
 * out of the cache (wrong numbers, never an out-of-bounds access).
 * Different chunking changes the fp32 summation order, so results with and
 * without hints agree up to rounding.
 * sfi_fast_step_noalloc and sfi_fast_step_compact ignore them. */
typedef struct sfi_kv {
  const uint16_t *k;
  const uint16_t *v;
  const int32_t *page_table;  /* NULL => contiguous */
  int32_t page_size;          /* paged only: power of two, 16..1024 */
  int32_t max_pages;          /* paged only: row stride of page_table */
  int32_t num_pages;          /* paged only: pages in the pool */
  const int32_t *seq_len;     /* [B] */
  int32_t B, Hq, Hkv, d;      /* d in {64, 128}; Hq % Hkv == 0; Hq/Hkv in {1,2,4,5,8} */
  int32_t cap;                /* contiguous only: rows per (b, kv head) */
  int32_t max_seq_len;        /* [host] */
  const uint16_t *k_new;      /* NULL, or the step's new rows [B][Hkv][d] (fused append) */
  const uint16_t *v_new;
  double *norm_stats;         /* NULL, or [B][Hkv][2] key-norm statistics (above) */
  int32_t norm_stats_valid;   /* [host] 1: norm_stats is current for the slow sequences */
  const int32_t *slow_len_host; /* [host] NULL, or the slow entries' seq_len (above) */
  const int32_t *fast_len_host; /* [host] NULL, or bounds on the fast entries' row lists */
} sfi_kv;

enum { SFI_SCORE_FUSED = 0, SFI_SCORE_RAW = 1 };

/* Selector parameters.  FUSED: score = evidence f, prior r from key norms
 * and positions, s = (1-lambda) f + lambda r  [SFI 3.B; fusion closed form in
 * the Korean summary, section 2.B].  RAW: the scores are ranked as given
 * (Vegas aggregated logits). */
typedef struct sfi_select_params {
  int32_t mode;       /* SFI_SCORE_FUSED or SFI_SCORE_RAW */
  float lambda;       /* [0, 1] */
  float norm_coef;    /* prior: weight of the standardised key norm (0.5) */
  float pos_tau;      /* prior: recency time constant in tokens (1024), > 0 */
  int32_t n_sink;     /* >= 0 */
  int32_t window;     /* >= 0 */
  int32_t k;          /* > 0: capacity (and row stride) of each index list */
  const int32_t *k_per_seq; /* device [B] or NULL: sequence b keeps at most
                               min(k_per_seq[b], k) keys (negative -> 0);
                               NULL: k for every sequence */
  /* Score refinements [SFI 3.B; the Portuguese summary, 2.B: Soft-NMS keeps
   * neighbouring, correlated keys from filling one head's budget; cross-head
   * exclusivity penalises the same key being picked by several heads].  The
   * pages give no formula; the reading implemented (all 0 = off):
   *   Soft-NMS: a candidate's log score drops by log(1/(1 - nms_alpha))
   *     once per candidate within nms_radius positions that ranks above it
   *     (larger score, or equal score and lower index); one pass.
   *   Exclusivity: after a first Top-K of every head row of a sequence, a
   *     row's key j loses log(1/(1 - excl_beta)) of log score once per other
   *     row whose first Top-K holds j, and the Top-K is taken again (two
   *     selection rounds; H >= 2 rows).
   * Both penalties act on log scores [SFI 3.B]: the FUSED score is a
   * probability, so a penalty of m log(1/(1 - a)) is the factor (1 - a)^m;
   * a RAW score (Vegas' summed logits) is already a log score of either
   * sign, so the penalty is subtracted from it.  Decisions use float32.
   * fused_out holds the score before either refinement.
   * nms_radius in [0, 8], nms_alpha and excl_beta in [0, 1) (else
   * SFI_ERR_RANGE).  sfi_decode_layer_step defers a selection into one key
   * and one pick pass, so it rejects excl_beta != 0 (SFI_ERR_UNSUPPORTED). */
  int32_t nms_radius;
  float nms_alpha;
  float excl_beta;
} sfi_select_params;

/* ---------------------------------------------------------------- sizes */

/* Workspace for sfi_slow_step on this cache (valid for any batch_n <= B). */
size_t sfi_slow_workspace_bytes(const sfi_kv *kv);
/* Workspace for sfi_select over B x H score rows of max length max_seq_len. */
size_t sfi_select_workspace_bytes(int32_t B, int32_t H, int32_t max_seq_len);
/* Workspace for sfi_fast_step with index lists of capacity sel_k. */
size_t sfi_fast_workspace_bytes(const sfi_kv *kv, int32_t sel_k, int32_t n_sink, int32_t window);
/* Workspace for sfi_verify_aggregate with T query rows per sequence. */
size_t sfi_verify_workspace_bytes(const sfi_kv *kv, int32_t T);

/* ---------------------------------------------------------------- calls */

/* Slow step [SFI 3.A slow steps, 3.B evidence]: dense attention of one decode
 * query per sequence over all seq_len[b] keys.
 *   q         [B][Hq][d] bf16; row b is used for each listed sequence b.
 *   out       [B][Hq][d] fp32: softmax(q K^T / sqrt(d)) V per head.
 *   evidence  [B][Hkv][ld] fp32 or NULL: f[b][g][j], j < seq_len[b], the
 *             softmax probability of key j averaged over the Hq/Hkv query
 *             heads of kv head g (sums to 1).  NULL => plain dense attention.
 *   key_norm  [B][Hkv][ld] fp32 or NULL: Euclidean norm of key j.
 *   ld        >= max_seq_len when evidence or key_norm is given.
 * Errors: NULL/SHAPE/RANGE/WORKSPACE before launch, HIP on launch failure. */
sfi_status sfi_slow_step(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                         const uint16_t *q, float *out, float *evidence, float *key_norm,
                         int32_t ld, void *ws, size_t ws_bytes, void *stream);

/* Selector [SFI 3.B; Vegas 2.A]: per listed sequence b and head row h < H,
 * pick the min(k_b, |C|) best keys of C = [n_sink, seq_len[b] - window) by
 * (score desc, index asc), with k_b = k or min(k_per_seq[b], k), and write
 * them ascending to sel_idx[b][h][0..count) (row stride k), padding to k
 * with -1; sel_count[b][h] = count.
 *   FUSED: score = evidence f [B][H][ld], key_norm [B][H][ld] (both over
 *          j < seq_len[b]).  Prior r_j = w_j / sum w, w_j = exp(-norm_coef
 *          z_j) (1 + exp(-(t - j) / pos_tau)), z_j = key norm standardised by
 *          its population mean and std over j < seq_len[b] (z = 0 if the std
 *          is 0), t = seq_len[b] - 1.  s = (1 - lambda) f + lambda r is ranked
 *          and, if fused_out != NULL, written to fused_out[b][h][j] for
 *          j < seq_len[b].
 *   RAW:   score [B][H][ld] is ranked as is (finite values; key_norm,
 *          lambda, norm_coef, pos_tau and fused_out are ignored).  Scores
 *          must be defined on all of C.
 * H is Hkv for per-head memories (SFI) or 1 for one head-shared list (Vegas).
 * max_seq_len <= 2,097,152 (else SFI_ERR_UNSUPPORTED).  NaN scores give an
 * unspecified (but in-range) selection. */
sfi_status sfi_select(const sfi_select_params *p, const int32_t *batch_ids, int32_t batch_n,
                      const int32_t *seq_len, int32_t B, int32_t H, int32_t max_seq_len,
                      const float *score, const float *key_norm, int32_t ld,
                      int32_t *sel_idx, int32_t *sel_count, float *fused_out,
                      void *ws, size_t ws_bytes, void *stream);

/* Cache append [SFI technical summary, section 1: every decode step attends
 * the whole cached history, which grows by the step's own key and value]:
 * for each listed sequence b, the T new rows k_new[b][t], v_new[b][t]
 * (t < T) are written to cache row j = seq_len[b] - T + t of every kv head
 * (seq_len already counts them; rows with j < 0 are skipped).  Paged caches
 * write through the page table.  k/v of *kv must be writable device memory.
 *   k_new, v_new  [B][T][Hkv][d] bf16 bits, 16-byte aligned.
 *   1 <= T <= max_seq_len (else SFI_ERR_RANGE).
 * Call it before the step that reads the rows, on the same stream.  Moves
 * 2 x 2 d bytes per row and kv head (read and write of K and V).  With
 * kv->norm_stats set, a second launch adds the rows' key norms to it. */
sfi_status sfi_append_kv(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                         const uint16_t *k_new, const uint16_t *v_new, int32_t T, void *stream);

/* Fast step [SFI 3.A fast steps; Vegas 2 drafting]: attention of one decode
 * query per sequence over the fast set of its kv head g, with n = seq_len[b]:
 *   [0, min(n_sink, n))  U  [max(n_sink, n - window), n)  U
 *   { sel_idx[b][hs][i] : i < sel_count[b][hs], n_sink <= j < n - window }
 * where hs = g if sel_heads == Hkv, hs = 0 if sel_heads == 1 (head-shared).
 * Entries outside that range (including -1 padding and keys now inside the
 * window) are skipped.  The listed entries of one list must be distinct.
 *   sel_idx [B][sel_heads][sel_k] int32, sel_count [B][sel_heads] int32.
 *   out     [B][Hq][d] fp32. */
sfi_status sfi_fast_step(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                         const uint16_t *q, const int32_t *sel_idx, const int32_t *sel_count,
                         int32_t sel_heads, int32_t sel_k, int32_t n_sink, int32_t window,
                         float *out, void *ws, size_t ws_bytes, void *stream);

/* sfi_fast_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, set, split plan and results (bit for bit) as
 * sfi_fast_step, minus the workspace: the split partials live in a
 * library-owned device array of SFI_NOALLOC_SCRATCH_BYTES per GPU, held
 * until the process ends.  The call allocates and frees nothing.
 *   Limit: the partials take batch_n * Hq * S * (d + 2) * 4 bytes (plus
 *   alignment), S the call's split count per (sequence, kv head) (about
 *   the GPU's resident workgroups / (batch_n * Hkv), at least 1); a call
 *   that needs more than SFI_NOALLOC_SCRATCH_BYTES returns
 *   SFI_ERR_WORKSPACE before anything is enqueued.
 *   The first call on each device resolves the array's device address
 *   (hipGetSymbolAddress, not a stream operation); make it outside a graph
 *   capture.  Every call on one GPU shares that GPU's array: calls that
 *   overlap in time on one GPU (other streams, other threads) race and give
 *   wrong results; order them.  Nothing in the array needs clearing: every
 *   planned partial is written before it is read. */
#define SFI_NOALLOC_SCRATCH_BYTES (16u << 20)
sfi_status sfi_fast_step_noalloc(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                 const uint16_t *q, const int32_t *sel_idx, const int32_t *sel_count,
                                 int32_t sel_heads, int32_t sel_k, int32_t n_sink, int32_t window,
                                 float *out, void *stream);

/* Compact copy of the selected rows [SFI 3.C and the Portuguese summary,
 * section 2.C: a fast kernel that reads the sink and selected rows from one
 * contiguous buffer instead of scattered cache rows]: for every sequence b of
 * the batch and kv head g, row i of ck / cv becomes the K / V row of key
 * j = sel_idx[b][hs][i], for i < min(sel_count[b][hs], sel_k) and
 * 0 <= j < seq_len[b] (hs as in sfi_fast_step); other rows are left as they
 * are.  Call it after a selection (the copy holds that selection's rows) and
 * before the fast steps that use it.
 *   ck, cv  [B][Hkv][sel_k][d] bf16 bits, 16-byte aligned (else
 *           SFI_ERR_RANGE); caller-owned.
 * Moves 2 x 2 d bytes per listed row (read and write of K and V). */
sfi_status sfi_compact_selected(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                const int32_t *sel_idx, const int32_t *sel_count, int32_t sel_heads,
                                int32_t sel_k, uint16_t *ck, uint16_t *cv, void *stream);

/* sfi_fast_step with the selected rows read from the compact copy made by
 * sfi_compact_selected from the same sel_idx / sel_count (sinks and window
 * still come from the cache).  Same set, same split plan and same order of
 * arithmetic as sfi_fast_step, so the results are equal bit for bit.  A
 * chunk of the row list made only of selected entries issues its first row
 * loads together with its query and index loads (the copy's addresses need
 * no index).  Arguments as sfi_fast_step, plus ck, cv as above; workspace
 * sfi_fast_workspace_bytes. */
sfi_status sfi_fast_step_compact(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                 const uint16_t *q, const int32_t *sel_idx, const int32_t *sel_count,
                                 int32_t sel_heads, int32_t sel_k, int32_t n_sink, int32_t window,
                                 const uint16_t *ck, const uint16_t *cv, float *out, void *ws,
                                 size_t ws_bytes, void *stream);

/* Slow step with a multi-query observation window [SFI 3.B: the evidence is
 * the attention observed in the slow step's window; here the window is the
 * last w decode queries of the sequence].  Row t (0..w-1) of q_win sits at
 * position n - w + t (n = seq_len[b]) and attends keys [0, n - w + t]:
 *   out[b][t][h]   that row's attention output (row w-1 is the decode step);
 *   evidence[b][g][j] = (1/(w G)) sum_t sum_{h of group g} p_t[h][j], j < n,
 *                  the rows' softmax probabilities (zero past a row's last
 *                  key) averaged over the window and the group: with w = 1
 *                  it is sfi_slow_step's evidence;
 *   key_norm[b][g][j] = ||k_j|| for j < n (optional).
 * Then sfi_select (FUSED) forms the selection as after sfi_slow_step.
 *   q_win [B][w][Hq][d] bf16; out [B][w][Hq][d] fp32; evidence, key_norm
 *   [B][Hkv][ld] fp32, ld >= max_seq_len; w <= max_seq_len.
 * Needs w * (Hq/Hkv) <= 32 and Hq/Hkv != 5 (SFI_ERR_UNSUPPORTED otherwise):
 * the w x G rows of a kv head are one 32-column MFMA tile.  The keys are read
 * twice (K, V for the outputs and the rows' softmax sums, then K again for
 * the evidence): 6 d bytes per key and kv head. */
size_t sfi_slow_window_workspace_bytes(const sfi_kv *kv, int32_t w);
sfi_status sfi_slow_step_window(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                const uint16_t *q_win, int32_t w, float *out, float *evidence,
                                float *key_norm, int32_t ld, void *ws, size_t ws_bytes, void *stream);

/* One decode step of a batch whose sequences take different paths [SFI 3.A
 * slow and fast steps; 3.C, which overlaps the slow path with fast steps]:
 * the slow step (dense attention with evidence) of slow_ids[0..n_slow) and the
 * fast step of fast_ids[0..n_fast), computed by one partial grid and one
 * finalize grid in which both sets of sequences share the chip.  The outputs
 * equal those of sfi_slow_step on slow_ids and sfi_fast_step on fast_ids, up to
 * floating-point rounding (the two calls split the rows differently).
 *   slow_ids, fast_ids  device int32 lists; together at most B ids, all
 *                       distinct (a sequence takes one path per step).
 *   evidence            required when n_slow > 0; key_norm optional.
 *   ws                  sfi_decode_step_workspace_bytes(kv, sel_k, n_sink, window).
 * Other arguments as in sfi_slow_step and sfi_fast_step.
 * Errors: as those two calls, and SFI_ERR_RANGE if n_slow + n_fast > B. */
size_t sfi_decode_step_workspace_bytes(const sfi_kv *kv, int32_t sel_k, int32_t n_sink,
                                       int32_t window);
sfi_status sfi_decode_step(const sfi_kv *kv, const int32_t *slow_ids, int32_t n_slow,
                           const int32_t *fast_ids, int32_t n_fast, const uint16_t *q, float *out,
                           float *evidence, float *key_norm, int32_t ld, const int32_t *sel_idx,
                           const int32_t *sel_count, int32_t sel_heads, int32_t sel_k,
                           int32_t n_sink, int32_t window, void *ws, size_t ws_bytes,
                           void *stream);

/* A decode step followed by the refresh of the slow sequences' selections
 * [SFI 3.A: a slow step refreshes the selected memory; 3.B: the selector runs
 * on the slow step's evidence and the cache statistics]: the outputs of
 * sfi_decode_step on slow_ids / fast_ids (per-head index lists of capacity
 * p->k, n_sink = p->n_sink, window = p->window), then the selections of
 * sfi_select (FUSED) for slow_ids written to sel_idx / sel_count.  The slow
 * step also forms the selector's prior statistics (key-norm mean and std,
 * prior-weight sums) while it has the key norms at hand, so the selection
 * starts at its key pass; results equal those of the separate calls up to
 * floating-point rounding (near-tie keys may differ).
 *   p           FUSED parameters (RAW -> SFI_ERR_RANGE); p->k_per_seq allowed.
 *   evidence, key_norm  required when n_slow > 0 ([B][Hkv][ld]).
 *   sel_idx, sel_count  read for fast_ids, written for slow_ids (disjoint).
 *   fused_out   [B][Hkv][ld] or NULL: the fused scores s of slow_ids.
 *   ws          sfi_decode_step_select_workspace_bytes(kv, p->k, p->n_sink,
 *               p->window) bytes.
 * Errors: as sfi_decode_step and sfi_select. */
size_t sfi_decode_step_select_workspace_bytes(const sfi_kv *kv, int32_t sel_k, int32_t n_sink,
                                              int32_t window);
sfi_status sfi_decode_step_select(const sfi_kv *kv, const sfi_select_params *p,
                                  const int32_t *slow_ids, int32_t n_slow, const int32_t *fast_ids,
                                  int32_t n_fast, const uint16_t *q, float *out, float *evidence,
                                  float *key_norm, int32_t ld, int32_t *sel_idx, int32_t *sel_count,
                                  float *fused_out, void *ws, size_t ws_bytes, void *stream);

/* A selection whose slow step has run and whose key and pick passes are
 * postponed: the cross-layer pipeline of sfi_decode_layer_step [SFI 3.C: the
 * slow path's selector is overlapped with other work].  Host struct, filled
 * by sfi_decode_layer_step (defer) and passed on unchanged; active = 0 means
 * nothing is pending.  The buffers it names (its layer's evidence, key norms,
 * index lists, fused scores, selector workspace and slow_ids list) must stay
 * untouched until the selection has run. */
typedef struct {
  int32_t active;
  sfi_select_params params;
  const int32_t *batch_ids;
  int32_t batch_n;
  const int32_t *seq_len;
  int32_t B, H, max_seq_len;
  const float *evidence;
  const float *key_norm;
  int32_t ld;
  int32_t *sel_idx;
  int32_t *sel_count;
  float *fused_out;
  void *ws;
  size_t ws_bytes;
} sfi_deferred;

/* sfi_decode_step_select for one layer of a stack, with the selections of
 * consecutive layers overlapped [SFI 3.C]: a layer's attention does not read
 * another layer's selection, so the key and pick passes of the previous
 * layer's slow sequences (`pending`) run inside this call's partial and
 * finalize grids.  With `defer` non-NULL this layer's own selection is not
 * run but described in *defer (active = 1 when n_slow > 0), for the next
 * layer's call or sfi_run_deferred; with `defer` NULL it runs at the end of
 * this call.  pending NULL or inactive and defer NULL: exactly
 * sfi_decode_step_select.  Results are those of sfi_decode_step_select per
 * layer, bit for bit.
 *   pending   must name other buffers than this call's (another layer's):
 *             the same selector workspace, index lists or evidence give
 *             SFI_ERR_RANGE; it is validated like sfi_select (FUSED only).
 *   Other arguments and the workspace: as sfi_decode_step_select.
 * The caller orders the layers on one stream; the pending selection's index
 * lists are complete when this call's work on the stream is. */
sfi_status sfi_decode_layer_step(const sfi_kv *kv, const sfi_select_params *p, const int32_t *slow_ids,
                                 int32_t n_slow, const int32_t *fast_ids, int32_t n_fast,
                                 const uint16_t *q, float *out, float *evidence, float *key_norm,
                                 int32_t ld, int32_t *sel_idx, int32_t *sel_count, float *fused_out,
                                 void *ws, size_t ws_bytes, const sfi_deferred *pending,
                                 sfi_deferred *defer, void *stream);
/* Runs a deferred selection on its own (the last layer's, or when the next
 * call is not a layer step).  d NULL: SFI_ERR_NULL; inactive: nothing. */
sfi_status sfi_run_deferred(const sfi_deferred *d, void *stream);

/* Verification with aggregated logits [Vegas 2, 2.A, 2.B, 3]: T query rows
 * per sequence; row t sits at position n - T + t (n = seq_len[b], which
 * already counts the T rows) and attends keys [0, n - T + t].
 *   q        [B][T][Hq][d] bf16.
 *   out      [B][T][Hq][d] fp32.
 *   agg      [B][ld] fp32: agg[b][i] = sum over rows t in row_mask and all
 *            Hq heads of the logit of key i, for i < n - T (the prefix).
 *   row_mask bit t selects row t: (1 << T) - 1 for all rows,
 *            1 | 1 << (T - 1) for Collect-2-Query.  Nonzero, < (1 << T).
 *   1 <= T and T * Hq / Hkv <= 32; ld >= max_seq_len - T. */
sfi_status sfi_verify_aggregate(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                const uint16_t *q, int32_t T, uint32_t row_mask, float *out,
                                float *agg, int32_t ld, void *ws, size_t ws_bytes, void *stream);

/* sfi_verify_aggregate with raw-logit emission, the collection that the
 * Vegas page sets its design against [Vegas 2.B and 3: writing the
 * pre-softmax logits of the verified queries out to memory costs bandwidth,
 * which Collect-2-Query limits to two rows]: the verify kernel writes the
 * collected rows' logits to HBM and a second pass sums them into agg.
 *   logits  [B][R][Hq][logits_ld] fp32, R = popcount(row_mask): entry
 *           (b, r, h, i) = q_{t,h} . k_i / sqrt(d) for the r-th collected row t
 *           (ascending) and prefix keys i < n - T; entries past the prefix
 *           are not written.  16-byte aligned; logits_ld >= max_seq_len - T.
 *   agg     as sfi_verify_aggregate (summed over rows, then heads, in a fixed
 *           order: equal to the in-kernel aggregate up to rounding).
 * Other arguments, workspace and errors as sfi_verify_aggregate.  Moves
 * R * Hq * (n - T) * 4 bytes more than it, written and read back. */
sfi_status sfi_verify_raw_logits(const sfi_kv *kv, const int32_t *batch_ids, int32_t batch_n,
                                 const uint16_t *q, int32_t T, uint32_t row_mask, float *out, float *agg,
                                 int32_t ld, float *logits, int32_t logits_ld, void *ws, size_t ws_bytes,
                                 void *stream);

/* Slow/fast schedule [SFI 3.A: slow at a semantic boundary or when the reuse
 * budget is spent] -- host only.  events [steps][B] [host] marks boundaries
 * (or any other slow trigger); slow [steps][B] [host] receives 1 where the
 * step is slow: step 0, every event, and every step that follows `budget`
 * consecutive fast steps (budget < 0: no budget). */
sfi_status sfi_schedule(const uint8_t *events, int32_t steps, int32_t B, int32_t budget,
                        uint8_t *slow);

/* Human-readable name of a status [host]. */
const char *sfi_status_string(sfi_status s);

/* Library version string [host].  0.2: sfi_kv carries the key-norm
 * statistics and the host row-count hints (its layout differs from 0.1's). */
const char *sfi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SFI_H */
