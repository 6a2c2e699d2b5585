// Host-side interface between the C ABI (sfi_abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sfi_common.hpp"

namespace sfi {

// Split-K planning: a (sequence, kv head) row range is cut into chunks of a
// multiple of kSplitGranule rows, at most kMaxSplits per pair.
constexpr int kSplitGranule = 32;
constexpr int kMaxSplits = 512;
#ifndef SFI_MAX_FAST_CHUNK
#define SFI_MAX_FAST_CHUNK 1024
#endif
constexpr int kMaxFastChunk = SFI_MAX_FAST_CHUNK;  // fast-step chunks stage their row ids in LDS
// A workgroup's fixed cost in the co-launch plans' makespan estimate, in
// rows: k waves cost k x (rows per workgroup + this).  Without it the
// estimate could prefer 14 waves of 32-row workgroups to 3 waves of 160
// rows (a 3.4K + 31 x 772-row step: 52 against 25 us).
#ifndef SFI_PLAN_BLOCK_COST
#define SFI_PLAN_BLOCK_COST 128
#endif
constexpr int kPlanBlockCost = SFI_PLAN_BLOCK_COST;
// Fewest rows per fast block of a co-launched step planned from per-entry
// row counts: each block pays an index -> page -> row prologue before its
// gathers stream.
#ifndef SFI_MIN_FAST_TABLE_CHUNK
#define SFI_MIN_FAST_TABLE_CHUNK 512
#endif
constexpr int kMinFastTableChunk = SFI_MIN_FAST_TABLE_CHUNK;
// Fewest rows per slow block of such a step when its plan takes several
// waves of resident blocks.
#ifndef SFI_MULTIWAVE_SLOW_CHUNK
#define SFI_MULTIWAVE_SLOW_CHUNK 2048
#endif
constexpr int kMultiWaveSlowChunk = SFI_MULTIWAVE_SLOW_CHUNK;
// Rows per workgroup of a dense or slow step at most.  Splits are planned
// from the longest sequence of the batch (its lengths are on the device), so
// without a cap a long sequence in a ragged batch gets a few huge chunks
// while the short ones' workgroups exit at once; capped, it takes more
// workgroups, which the dispatcher runs in further waves.
#ifndef SFI_MAX_SLOW_CHUNK
#define SFI_MAX_SLOW_CHUNK 8192
#endif
constexpr int kMaxSlowChunk = SFI_MAX_SLOW_CHUNK;
// Keys per workgroup of the evidence pass.
constexpr int kEvidChunk = 2048;

// Plan of a split-K decode launch.
struct SplitPlan {
  int chunk;   // rows per workgroup
  int splits;  // workgroups per (sequence, kv head) for the host bound
  int stride;  // split stride of the partial buffers (>= splits)
};

// Partial-buffer stride (splits per pair) that covers L rows.
inline int split_stride(long long L) {
  long long s = (L + kSplitGranule - 1) / kSplitGranule;
  if (s < 1) s = 1;
  return s > kMaxSplits ? kMaxSplits : (int)s;
}

// Chunking of L rows per pair over `pairs` pairs so that one launch fills
// `slots` resident workgroups once, within the stride and a chunk cap; with
// whole_waves, a capped plan takes a whole number of such waves.
SplitPlan plan_splits(long long L, int pairs, int slots, int stride, int max_chunk, bool whole_waves);
// Chunking of L rows with about R rows per workgroup (multiple of the granule).
SplitPlan plan_rows(long long L, int stride, long long R, int max_chunk);

// Compute units of the current device (cached per device).
int device_cu_count();

struct SelRowMeta;
struct SelectLaunch;

struct AttnLaunch {
  KVView kv;
  const int32_t *seq_len;
  const int32_t *batch_ids;
  int batch_n;
  int B, Hq, Hkv, d, G;
  int max_len;
  bool paged;
  const uint16_t *q;
  float *out;
  // partials, indexed by sequence slot b: o [B][Hq][stride][d], ml [B][Hq][stride][2]
  float *part_o;
  float *part_ml;
  SplitPlan plan;
  // slow-step side outputs
  float *logits;      // [B][Hkv][lld][G] (log2-scaled), workspace
  int lld;
  float *evidence;    // [B][Hkv][ld] or nullptr
  float *key_norm;    // [B][Hkv][nld] or nullptr
  int ld;
  int nld;            // row stride of key_norm (ld, or max_len for workspace rows)
  // fast step
  const int32_t *sel_idx;
  const int32_t *sel_count;
  int sel_heads, sel_k, n_sink, window;
  // The selector's prior, computed by a slow step for the selection that
  // follows it (null nsum: not computed): per-split key-norm sums
  // [B][Hkv][stride][2] (workspace), and the selector workspace's per-chunk
  // prior-weight sums, row constants and bucket histograms it fills.
  double *nsum;
  float norm_coef, pos_tau;
  double *sel_wsum;      // [B*Hkv][selP]
  SelRowMeta *sel_meta;  // [B*Hkv]
  uint32_t *sel_ghist;   // [B*Hkv][4096]
  int selP;
  // Prior from the key-norm statistics kv.nstat instead of the per-split
  // sums (stats, nsum null): the partial kernel forms the row constants,
  // the splits' prior-weight sums wpart [B*Hkv][stride] and the updated
  // statistics nnext [B*Hkv][2], and the finalize stores those and runs the
  // key pass of keysel (non-null with stats) on the fused scores.
  bool stats;
  double *wpart;
  double *nnext;
  const SelectLaunch *keysel;
  // fast step: compact copy of the selected rows [B][Hkv][sel_k][d] (or null)
  const uint16_t *ck, *cv;
  // partial buffers indexed by batch entry (rows [batch_n][Hq][stride])
  // instead of by sequence id (rows [B][Hq][stride])
  bool part_by_entry;
  // plan fixed by the caller (launch_fast only): `plan` is used as given
  bool planned;
  // [host] the listed entries' row counts (slow and dense: the sequence
  // length; fast: a bound on the row list's length), in list order, or
  // null.  Set, the launchers plan the grid from them (a work table: no
  // block past an entry's rows) instead of from max_len.
  const int32_t *len_host;
  WorkTable wt;  // filled by the launcher
};

hipError_t launch_slow(const AttnLaunch &a, hipStream_t st);
hipError_t launch_fast(const AttnLaunch &a, hipStream_t st);
// The split plan launch_fast takes for `a` (chunk and split count; the
// stride is a.plan.stride's cap).
SplitPlan plan_fast(const AttnLaunch &a);
// Fast step whose selected rows come from the compact copy a.ck / a.cv.
hipError_t launch_fast_compact(const AttnLaunch &a, hipStream_t st);
// Copy the K/V rows of every valid selected entry (i < count, 0 <= id < n)
// to row i of the compact copy ck / cv ([B][Hkv][sel_k][d]).
hipError_t launch_compact(const AttnLaunch &a, uint16_t *ck, uint16_t *cv, hipStream_t st);
// Write T new K/V rows per listed sequence at cache rows seq_len - T + t.
hipError_t launch_append(const AttnLaunch &a, const uint16_t *k_new, const uint16_t *v_new, int T,
                         hipStream_t st);
struct SelectLaunch;
// Slow step with evidence (sa) and fast step (fa) on disjoint sequences,
// co-launched; either share may be empty.  A non-null pend is a selection
// of other buffers (another layer's, its prior already formed by its slow
// step) whose key and pick passes run in this step's two grids.
hipError_t launch_step(const AttnLaunch &sa, const AttnLaunch &fa, hipStream_t st,
                       const SelectLaunch *pend = nullptr);

constexpr int kSelChunk = 2048;       // keys per selector chunk workgroup
constexpr int kNmsMaxRadius = 8;      // Soft-NMS neighbourhood (halo staged in LDS)
constexpr int kSelMaxChunks = 1024;   // chunks per row
constexpr int kSelMaxLen = kSelChunk * kSelMaxChunks;  // longest row: 2,097,152 keys

// Per-row prior constants shared by the selector's kernels.
struct SelRowMeta {
  float muf, cz;           // mean key norm, -norm_coef log2(e) / std
};

// Selector workspace, carved from the caller's buffer.
struct SelWork {
  int P;                      // chunks per row
  uint32_t *ghist;            // [rows][4096] bucket histogram of the row
  uint16_t *cum;              // [rows][P][4096] per chunk: keys in buckets >= b
  unsigned long long *sorted; // [rows][P][kSelChunk] bucket-sorted composites
  double *nsum;               // [rows][P][2] key-norm sums per chunk
  double *wsum;               // [rows][P] prior-weight sums per chunk
  SelRowMeta *meta;           // [rows]
};

struct SelectLaunch {
  int mode;
  float lambda, norm_coef, pos_tau;
  int n_sink, window, k;
  const int32_t *k_seq;  // [B] per-sequence list length (clamped to k) or null
  const int32_t *batch_ids;
  int batch_n;
  const int32_t *seq_len;
  int B, H, max_seq_len;
  const float *score;
  const float *key_norm;
  int ld;
  int32_t *sel_idx;
  int32_t *sel_count;
  float *fused_out;   // [B][H][fo_ld] or null
  int fo_ld;
  bool prior_done;    // the slow step already wrote wsum, meta and cleared ghist
  SelWork ws;
  // Soft-NMS (radius 0: off) and cross-head exclusivity (beta 0: off)
  int nms_radius;
  float nms_alpha;
  float excl_beta;
  // exclusivity's second round: per-key count of rows whose first Top-K
  // holds it [B][ld32 * 32] and each row's membership bits [B*H][ld32]
  // (ld32 * 32 = whole chunks), and the second round's row histograms
  // [B*H][4096]
  uint32_t *excl_cnt;
  uint32_t *excl_bits;
  uint32_t *excl_ghist;
  int ld32;
  int round;  // 1: exclusivity's second key pass (applies the penalty)
};

hipError_t launch_select(const SelectLaunch &a, hipStream_t st);
// The pick pass alone, for a selection whose key pass already ran.
hipError_t launch_pick(const SelectLaunch &a, hipStream_t st);

struct VerifyLaunch {
  KVView kv;
  const int32_t *seq_len;
  const int32_t *batch_ids;
  int batch_n;
  int B, Hq, Hkv, d, G, T;
  int max_seq_len;
  bool paged;
  uint32_t row_mask;
  const uint16_t *q;
  float *out;
  float *agg;
  int ld;
  float *part_o;      // [B][T*Hq][stride][d]
  float *part_ml;     // [B][T*Hq][stride][2]
  float *part_agg;    // [B][Hkv][lld], or null (observation-window slow step)
  int lld;
  SplitPlan plan;
  // observation-window slow step: per-row (reference, sum) [B][T*Hq][2]
  // (workspace) and the evidence / key norms [B][Hkv][ld] it writes
  float *rstat;
  float *evidence;
  float *key_norm;
  // raw-logit emission (or null): [B][popcount(row_mask)][Hq][raw_ld]
  float *raw;
  int raw_ld;
};

hipError_t launch_verify(const VerifyLaunch &a, hipStream_t st);
// Keys per wave of the verify kernel: the workgroups of B x Hkv pairs fill
// the device's resident slots in whole rounds.
int verify_chunk_for(int B, int Hkv, int max_seq_len, int d, int G);
// Partial slots per (row, sequence) of the verify kernel for keys per wave `chunk`.
int verify_stride_for(int max_seq_len, int chunk);

}  // namespace sfi
