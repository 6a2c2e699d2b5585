// Split-K decode attention for one query per sequence on gfx950.
//
// Slow step (Slow-Fast Inference, technical summary section 3.A: a slow step
// runs dense attention over the whole cached history; section 3.B: its
// attention is the selector's evidence): every cached key of a (sequence, kv
// head) pair is visited once.  Fast step (section 3.A: attention restricted to
// sink tokens, the recent window and the selected memory; the Portuguese
// summary, section 2.A, notes that its cost tracks the sparse-state size, not
// the context): the same inner loop over a gathered row list.
//
// Layout and mapping (HBM-bound GEMV, no MFMA):
//   * a key/value row of d bf16 is read by d/8 lanes, 16 bytes each, so one
//     wave instruction covers 4 (d=128) or 8 (d=64) consecutive rows and a
//     workgroup of 256 threads streams 16/32 rows per instruction;
//   * each lane keeps the G query heads of its kv head for its 8 dimensions,
//     forms G partial dot products with v_dot2_f32_bf16 and reduces them
//     across its lane group with DPP row permutes;
//   * every lane group runs its own fp32 online softmax (log2 domain) over the
//     rows it owns; groups are merged with cross-lane shuffles, waves through
//     LDS, and the workgroup writes one (m, Z, O) partial per query head;
//   * a finalize kernel merges the partials in a fixed order and, for slow
//     steps, turns the per-key logits written on the way into the evidence
//     f_j = (1/G) sum_h p_hj.
#include <algorithm>
#include <type_traits>

#include "sfi_internal.hpp"
#include "select_body.hpp"

namespace sfi {
namespace {

// Rows per lane group and pipeline stage (0: LPR / 8, i.e. 8 rows per wave
// per stage whatever the lane-group width; measured faster than 16 at the
// 32K and 128K G = 4 shapes, whose workgroups then start consuming sooner
// and finish with a shorter last stage).
#ifndef SFI_DECODE_U
#define SFI_DECODE_U 0
#endif
// Fast-step launch shape (rows per stage, lanes per row; 0 = the automatic
// choice) and lanes per row for dense/slow steps.
#ifndef SFI_FAST_U
#define SFI_FAST_U SFI_DECODE_U
#endif
#ifndef SFI_FAST_LPR
#define SFI_FAST_LPR 0
#endif
#ifndef SFI_DENSE_LPR
#define SFI_DENSE_LPR 0
#endif
// Dims of a key row held by lane `sub` of its lane group: line-major (1) puts
// the lane's c-th 16-byte slice in the c-th 128-byte line of the row, so one
// load instruction of the group reads whole lines; 0 gives each lane one
// contiguous run of D/LPR dims.
#ifndef SFI_LINE_MAJOR
#define SFI_LINE_MAJOR 1
#endif
#ifndef SFI_WAVES_OF_WG
#define SFI_WAVES_OF_WG 1
#endif


enum { MODE_SLOW = 0, MODE_FAST = 1 };
constexpr int kThreads = 256;

struct PartialArgs {
  KVView kv;
  int B, max_len;
  const int32_t *seq_len;
  const int32_t *batch_ids;
  const uint16_t *q;
  int Hq;
  int chunk;
  int stride;
  float *part_o;
  float *part_ml;
  float *logits;
  int lld;
  float *key_norm;  // evidence mode: never null (workspace rows when the caller passes none)
  int ld;
  int nld;          // row stride of key_norm
  const int32_t *sel_idx;
  const int32_t *sel_count;
  int sel_heads, sel_k, n_sink, window;
  float qscale;  // log2(e) / sqrt(d)
  double *nsum;  // [B][Hkv][stride][2] per-split key-norm sums, or null
  // fast step: compact copy of the selected rows, [B][Hkv][sel_k][D] (or null)
  const uint16_t *ck, *cv;
  int pe;  // 1: partial buffers indexed by batch entry instead of sequence id
  // Evidence mode with the prior formed from the key-norm statistics
  // (the STATS kernels; nsum null): mean and std of the row's key norms from
  // kv.nstat (plus the step's own row when it is appended here), each
  // split's sum of the prior weights into wpart [B*Hkv][stride] (fp64), the
  // row constants into sel_meta and the updated statistics into nnext
  // [B*Hkv][2] (split 0; the finalize stores them), and the splits clear
  // the row's bucket histogram sel_ghist between them for the key pass in
  // the finalize.
  double *wpart;
  double *nnext;
  SelRowMeta *sel_meta;
  uint32_t *sel_ghist;
  int nsp;  // planned splits per (sequence, kv head)
  WorkTable wt;  // per-entry split counts (wt.n = 0: nsp for every entry)
  float norm_coef, pos_tau;
};

// Maximum over the wave of a value that is equal within each aligned group
// of 8 lanes (xor 8 stays inside a 16-lane row: a DPP rotate).
__device__ __forceinline__ float wave_max_groups(float x) {
  x = fmaxf(x, dpp_f32<0x128>(x));  // row_ror:8 == lane ^ 8 within a row
  x = xmax<16>(x);
  x = xmax<32>(x);
  return x;
}

// Fast-step row list of (b, g): [sinks | window | selected].
struct FastList {
  int ns, w0, nw, cnt;
  const int32_t *sel;
  __device__ int length() const { return ns + nw + cnt; }
};

__device__ __forceinline__ FastList fast_list(const int32_t *sel_idx, const int32_t *sel_count,
                                              int sel_heads, int sel_k, int n_sink, int window,
                                              int b, int g, int n) {
  FastList f;
  f.ns = min(n_sink, n);
  f.w0 = max(n_sink, n - window);
  f.nw = max(0, n - f.w0);
  const int hs = (sel_heads == 1) ? 0 : g;
  const int c = sel_count[b * sel_heads + hs];
  f.cnt = min(max(c, 0), sel_k);
  f.sel = sel_idx + ((size_t)b * sel_heads + hs) * sel_k;
  return f;
}

// One workgroup's share of a decode step: rows [split*chunk, ...) of the row
// list of (sequence batch_ids[zb], kv head g).  A device function so that the
// co-launch kernel below can run slow and fast shares in one grid.
template <int D, int G, bool PAGED, int MODE, bool EVID, bool COMPACT = false, bool STATS = false>
__device__ __forceinline__ void partial_body(const PartialArgs &a, int split, int g, int zb) {
  static_assert(!STATS || EVID, "the statistics prior is an evidence-mode variant");
  // 8 lanes per row halves the cross-lane reduction and softmax work per row
  // compared with 16; wide groups (G*D >= 640) use 16 to bound accumulators
  // (at G = 5, d = 128 eight lanes would need all 256 VGPRs).
  constexpr int LPR_AUTO = (G * D >= 640) ? 16 : 8;
  constexpr int LPR_SET = (MODE == MODE_FAST) ? SFI_FAST_LPR : SFI_DENSE_LPR;
  constexpr int LPR = (LPR_SET == 8 || (LPR_SET == 16 && D == 128)) ? LPR_SET : LPR_AUTO;  // lanes per row
  constexpr int DPL = D / LPR;         // dims per lane (8 or 16)
  constexpr int NV = DPL / 8;          // 16-byte slices per row per lane
  constexpr int RPB = kThreads / LPR;  // rows per workgroup instruction
  constexpr int U_SET = (MODE == MODE_FAST) ? SFI_FAST_U : SFI_DECODE_U;
  constexpr int U = U_SET > 0 ? U_SET : LPR / 8;  // rows per lane group per stage
  constexpr int NW = kThreads / 64;
  // Lazy rescaling: the running reference m only moves when a logit exceeds
  // it by more than kSlack (log2 units), so p = 2^(l - m) stays <= 2^kSlack.
  // m is the same in every lane of the wave (it moves to the wave's maximum),
  // so the lane groups' partials merge below by plain addition.
  constexpr float kSlack = 8.0f;

  __shared__ int s_idx[MODE == MODE_FAST ? kMaxFastChunk : 1];
  // Paged caches: the physical page of each row the chunk reads, resolved
  // once into LDS (fast: one per list entry; dense/slow: one per page of the
  // chunk's contiguous rows, chunks of at most kMaxSlowChunk rows and pages
  // of at least 16), so the main loop's row addresses need no global load:
  // a page-table load issued behind a stage's row loads would make its wait
  // drain them too, leaving one stage in flight.
  constexpr int kPgSlots = (MODE == MODE_FAST) ? kMaxFastChunk : kMaxSlowChunk / 16 + 2;
  __shared__ int s_pg[PAGED ? kPgSlots : 1];
  __shared__ float s_m[NW][G], s_z[NW][G];
  __shared__ float s_acc[NW][G][D];
  // Evidence staging: the logits (G per key) and norms of one block of
  // kEvBlock consecutive rows, written out when the block is complete.
  constexpr bool EV_LDS = EVID;
  constexpr int kEvBlock = 512;
  __shared__ float s_evl[EV_LDS ? kEvBlock * G : 1];
  __shared__ float s_evn[EV_LDS ? kEvBlock : 1];

  const int b = batch_seq(a.batch_ids, zb, a.B);
  if (b < 0) return;
  const int tid = threadIdx.x;
  const int p0 = split * a.chunk;
  const int sub = tid % LPR;
  const int rg = tid / LPR;
  // element offset in the row of this lane's c-th 16-byte slice
  auto slice = [&](int c) { return SFI_LINE_MAJOR ? c * LPR * 8 + sub * 8 : sub * DPL + 8 * c; };

  // Loads that need only the sequence id go out before the sequence length
  // and the list length are known, so they share one round trip with them:
  // the query slices and, for the fast step, the chunk's index entries at the
  // positions they take when the fixed part (sinks + window) is full, which
  // is every sequence longer than n_sink + window; a shorter sequence loads
  // them again below.  Entries are clamped to the list's row (sel_k), so every
  // load stays inside it; entries past the list's length are never used.
  uint32_t qv[G][4 * NV];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const uint4 t = ldg16(a.q + ((size_t)b * a.Hq + g * G + h) * D + slice(c));
      qv[h][4 * c + 0] = t.x; qv[h][4 * c + 1] = t.y; qv[h][4 * c + 2] = t.z; qv[h][4 * c + 3] = t.w;
    }
  }
  constexpr int IPT = (MODE == MODE_FAST) ? kMaxFastChunk / kThreads : 1;
  int jv[IPT];
  const int nfix_full = a.n_sink + a.window;
  const size_t lrow = (size_t)(b * a.kv.Hkv + g);
  // Prior from the key-norm statistics: the row's sums and (fused append)
  // the slices of the step's own K row go out with the query loads and
  // have arrived once the sequence length has.
  double st1 = 0.0, st2 = 0.0;
  uint4 knx = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (STATS) {
    {
      st1 = a.kv.nstat[lrow * 2 + 0];
      st2 = a.kv.nstat[lrow * 2 + 1];
      if (a.kv.k_new != nullptr) knx = ldg16(a.kv.k_new + lrow * D + 8 * ((tid & 63) % (D / 8)));
    }
  }

  // One pipeline stage: U rows per lane group, K and V slices of DPL dims.
  struct Stage {
    uint4 k[U][NV], v[U][NV];
    int j[U];   // key id, -1 for a masked row
    int js[U];  // dense/slow: the row actually read (a masked row reads the chunk's last row)
  };
  // Compact rows: list position p >= nfix is entry p - nfix of the selection,
  // row p - nfix of the compact copy; the address needs no index, so a chunk
  // made only of selected entries issues its first stage with the query
  // loads (taking nfix = n_sink + window, every sequence longer than that)
  // and fills the rows' key ids in once the list is staged.
  auto load_compact = [&](Stage &st, int base, int nfix) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(max(base + u * RPB - nfix, 0), a.sel_k - 1);
      const size_t off = (lrow * a.sel_k + i) * D;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        st.k[u][c] = ldg16_stream(a.ck + off + slice(c));
        st.v[u][c] = ldg16_stream(a.cv + off + slice(c));
      }
    }
  };
  Stage sa, sb;
  const bool spec_c = COMPACT && p0 >= nfix_full;  // chunk inside the selected part (if n is long)
  if constexpr (COMPACT) {
    if (spec_c) load_compact(sa, p0 + rg, nfix_full);
  }
  if constexpr (MODE == MODE_FAST) {
    const int32_t *srow =
        a.sel_idx + ((size_t)b * a.sel_heads + (a.sel_heads == 1 ? 0 : g)) * a.sel_k;
#pragma unroll
    for (int i = 0; i < IPT; ++i)
      jv[i] = (a.sel_k > 0) ? srow[min(max(p0 + tid + i * kThreads - nfix_full, 0), a.sel_k - 1)] : -1;
  }

  const int n = clamp_len(a.seq_len, b, a.max_len);
  // the prior's row constants (mean and std of the key norms, the step's
  // own row included), uniform over the workgroup and so held in scalar
  // registers through the main loop
  float st_muf = 0.f, st_cz = 0.f, st_ct = 0.f;
  if constexpr (STATS) {
    {
      if (a.kv.k_new != nullptr) {
        const float nu = wave_row_norm<D>(knx);
        st1 += (double)nu;
        st2 = fma((double)nu, (double)nu, st2);
      }
      prior_consts(st1, st2, n, a.norm_coef, &st_muf, &st_cz);
      st_muf = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(st_muf)));
      st_cz = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(st_cz)));
      st_ct = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(kLog2e / a.pos_tau)));
      if (tid == 0 && split == 0) {
        a.sel_meta[lrow].muf = st_muf;
        a.sel_meta[lrow].cz = st_cz;
        a.nnext[lrow * 2 + 0] = st1;
        a.nnext[lrow * 2 + 1] = st2;
      }
    }
  }
  int L = n;
  FastList fl;
  if constexpr (MODE == MODE_FAST) {
    fl = fast_list(a.sel_idx, a.sel_count, a.sel_heads, a.sel_k, a.n_sink, a.window, b, g, n);
    L = fl.length();
  }
  // Fused append: row n - 1 is this step's own key and value, at list
  // position app_p (-1 when the list does not hold it: a fast list without
  // a window).  The one workgroup whose chunk holds that position (the
  // first split when none does) reads the row from kv.k_new / kv.v_new in
  // the one stage that covers it, so no workgroup of this launch reads that
  // cache row, and stores it into the cache as it ends.
  constexpr int kAppSlices = D / 8;  // 16-byte slices per row
  const size_t new_row = lrow * D;
  int app_p = -1;
  bool app_wg = false;  // uniform over the workgroup
  if (a.kv.k_new != nullptr && n > 0) {
    app_p = n - 1;
    if constexpr (MODE == MODE_FAST) app_p = (fl.nw > 0) ? fl.ns + fl.nw - 1 : (n - 1 < fl.ns ? n - 1 : -1);
    app_wg = (app_p >= 0) ? (app_p >= p0 && app_p < p0 + a.chunk) : (split == 0);
  }
  // With key-norm statistics and no prior formed here (whose finalize
  // stores them), the row's norm is added to them.
  auto append_store = [&]() {
    if (app_wg) {
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (tid < 2 * kAppSlices) {
        const bool isv = tid >= kAppSlices;
        const int c = tid % kAppSlices;
        x = ldg16((isv ? a.kv.v_new : a.kv.k_new) + new_row + 8 * c);
        uint16_t *dst = const_cast<uint16_t *>(isv ? a.kv.v : a.kv.k);
        *reinterpret_cast<uint4 *>(dst + kv_row<D, PAGED>(a.kv, b, g, n - 1) + 8 * c) = x;
      }
      if (!STATS && a.kv.nstat != nullptr && a.nsum == nullptr && tid < 64) {  // wave 0: lanes 0 .. D/8 - 1 hold K
        const float nu = wave_row_norm<D>(x);
        if (tid == 0) {
          a.kv.nstat[lrow * 2 + 0] += (double)nu;
          a.kv.nstat[lrow * 2 + 1] = fma((double)nu, (double)nu, a.kv.nstat[lrow * 2 + 1]);
        }
      }
    }
  };
  if constexpr (STATS) {
    {  // this split's stripe of the row histogram
      const int nsp = entry_splits(a.wt, zb, a.nsp);
      for (int i = split * kThreads + tid; i < 4096; i += nsp * kThreads) a.sel_ghist[lrow * 4096 + i] = 0u;
    }
  }
  if (p0 >= L) {
    if constexpr (STATS) {
      if (tid == 0) a.wpart[lrow * a.stride + split] = 0.0;
    }
    append_store();
    // no rows here: a neutral partial (Z = 0), so the finalize can merge
    // every planned split without reading the list length
    if (tid < G) {
      const size_t slot = ((size_t)(a.pe ? zb : b) * a.Hq + g * G + tid) * a.stride + split;
      a.part_ml[slot * 2 + 0] = kNegBig;
      a.part_ml[slot * 2 + 1] = 0.f;
    }
    return;
  }
  const int p1 = min(L, p0 + a.chunk);

  if constexpr (MODE == MODE_FAST) {
    // Every list entry of the chunk is loaded before any is stored, so the
    // index loads are in flight together (one round trip instead of one per
    // 256 entries).
    const int nfix = fl.ns + fl.nw;
    if (nfix != nfix_full) {  // short sequence: the fixed part is shorter
#pragma unroll
      for (int i = 0; i < IPT; ++i)
        jv[i] = (fl.cnt > 0) ? fl.sel[min(max(p0 + tid + i * kThreads - nfix, 0), fl.cnt - 1)] : -1;
    }
    int jr[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int p = p0 + tid + i * kThreads;
      int j = -1;
      if (p < fl.ns) {
        j = p;
      } else if (p < nfix) {
        j = fl.w0 + (p - fl.ns);
      } else {
        j = jv[i];
        if (j < a.n_sink || j >= fl.w0) j = -1;  // padding, sink or now in window
      }
      jr[i] = j;
    }
    if constexpr (PAGED) {
      // every entry's page-table load in flight together (j < n <= the
      // table's rows; a skipped entry looks up page 0)
      int pgv[IPT];
#pragma unroll
      for (int i = 0; i < IPT; ++i)
        pgv[i] = a.kv.page_table[(size_t)b * a.kv.max_pages + (max(jr[i], 0) >> a.kv.page_shift)];
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        const int p = p0 + tid + i * kThreads;
        if (p < p1) s_pg[p - p0] = pgv[i];
      }
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int p = p0 + tid + i * kThreads;
      if (p < p1) s_idx[p - p0] = jr[i];
    }
    __syncthreads();
  } else if constexpr (PAGED) {
    // pages of the chunk's rows [p0, p1)
    const int pb = p0 >> a.kv.page_shift;
    const int npg = ((p1 - 1) >> a.kv.page_shift) - pb + 1;
    constexpr int PR = (kPgSlots + kThreads - 1) / kThreads;
    int pgv[PR];
#pragma unroll
    for (int r = 0; r < PR; ++r) {
      const int i = tid + r * kThreads;
      pgv[r] = (i < npg) ? a.kv.page_table[(size_t)b * a.kv.max_pages + pb + i] : 0;
    }
#pragma unroll
    for (int r = 0; r < PR; ++r) {
      const int i = tid + r * kThreads;
      if (i < npg && i < kPgSlots) s_pg[i] = pgv[r];
    }
    __syncthreads();
  }


  float m[G], Z[G], acc[G][DPL];
  double ns1 = 0.0, ns2 = 0.0;  // key-norm sums of this lane's rows (evidence mode; STATS: prior-weight sum)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    Z[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
  }

  // Every lane issues its loads unconditionally: a row past the chunk or a
  // skipped list entry reads row 0 of the same (sequence, kv head), which
  // exists whenever the list is non-empty, and is masked out in consume().
  // Loads that sit behind a per-lane branch would leave the number of loads
  // in flight unknown at compile time, and every later wait would have to
  // drain all of them, collapsing the two-stage pipeline.
  auto load_stage = [&](Stage &st, int base) {
    // Can a lane of this stage read the step's own row (fused append)?
    // Uniform: the stage holding its list position and every later one (a
    // masked dense row re-reads the chunk's last row, which is that row in
    // the last chunk, and its evidence values must be the row's own).
    const int sbase = __builtin_amdgcn_readfirstlane(base - rg);
    const bool st_fresh = app_wg && app_p >= 0 && app_p < sbase + RPB * U;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + u * RPB;
      int j, jr;
      if constexpr (MODE == MODE_FAST) {
        j = s_idx[min(p - p0, a.chunk - 1)];
        j = (p < p1) ? j : -1;
        jr = max(j, 0);
      } else {
        // a masked lane reads the chunk's last row, so the logits and norm it
        // stores in evidence mode are that row's own (see consume())
        j = (p < p1) ? p : -1;
        jr = min(p, p1 - 1);
      }
      st.j[u] = j;
      st.js[u] = jr;
      size_t off;
      if constexpr (PAGED) {
        const int sh = a.kv.page_shift;
        int pg;
        if constexpr (MODE == MODE_FAST) pg = s_pg[min(p - p0, a.chunk - 1)];
        else pg = s_pg[min((jr >> sh) - (p0 >> sh), kPgSlots - 1)];
        pg = min(max(pg, 0), a.kv.num_pages - 1);
        off = ((((size_t)pg * a.kv.Hkv + g) << sh) + (size_t)(jr & ((1 << sh) - 1))) * D;
      } else {
        off = kv_row<D, false>(a.kv, b, g, jr);
      }
      const uint16_t *kp = a.kv.k + off, *vp = a.kv.v + off;
      if (st_fresh) {  // the step's own row comes from the new-row buffers
        const bool f = jr == n - 1;
        kp = f ? a.kv.k_new + new_row : kp;
        vp = f ? a.kv.v_new + new_row : vp;
      }
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        // Rows are loaded with the non-temporal hint.  Cold, back to back,
        // it measured faster in every mode: 8 sequences at 32K, dense 188 ->
        // 170 us, dense with evidence 236 -> 216 us (the logits it writes
        // and the finalize reads back are no longer pushed out by the row
        // stream), fast 23.8 -> 22.5 us (warm too: 21.2 -> 20.8 us).
        st.k[u][c] = ldg16_stream(kp + slice(c));
        st.v[u][c] = ldg16_stream(vp + slice(c));
      }
    }
  };
  auto consume = [&](const Stage &st) {
    float l[U][G], lr[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sdot = 0.f;
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          sdot = dot2_bf16(qv[h][4 * c + 0], st.k[u][c].x, sdot);
          sdot = dot2_bf16(qv[h][4 * c + 1], st.k[u][c].y, sdot);
          sdot = dot2_bf16(qv[h][4 * c + 2], st.k[u][c].z, sdot);
          sdot = dot2_bf16(qv[h][4 * c + 3], st.k[u][c].w, sdot);
        }
        sdot = group_sum<LPR>(sdot);
        lr[u][h] = sdot * a.qscale;
        l[u][h] = (st.j[u] >= 0) ? lr[u][h] : -INFINITY;
      }
    }
    if constexpr (EVID) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float nn = 0.f;
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          nn = dot2_bf16(st.k[u][c].x, st.k[u][c].x, nn);
          nn = dot2_bf16(st.k[u][c].y, st.k[u][c].y, nn);
          nn = dot2_bf16(st.k[u][c].z, st.k[u][c].z, nn);
          nn = dot2_bf16(st.k[u][c].w, st.k[u][c].w, nn);
        }
        nn = group_sum<LPR>(nn);
        // Every lane stores, with no branch: on gfx950 stores share the
        // vector-memory counter with loads, and a store the compiler cannot
        // count (one behind a per-lane branch) makes the next stage's wait
        // drain it too.  Lanes past the group's G heads repeat a head's
        // logit, every lane of the group stores the same norm, and a masked
        // row rewrites the chunk's last row with that row's own values.
        const int js = st.js[u];
        float v = lr[u][0];
#pragma unroll
        for (int h = 1; h < G; ++h) v = (sub % G == h) ? lr[u][h] : v;
        // the hardware square root (within 1 ulp; the library's sqrtf adds
        // a ~15-instruction correctly rounded refinement per key)
        const float nv = __builtin_amdgcn_sqrtf(nn);
        // row js sits in the current block (a masked row repeats the
        // chunk's last row, which is in the chunk's last block)
        const int r = (js - p0) & (kEvBlock - 1);
        s_evl[r * G + sub % G] = v;
        s_evn[r] = nv;
        if constexpr (!STATS) {
          if (a.nsum) {  // wave-uniform: only a step that forms the prior needs the sums
            const bool acc = st.j[u] >= 0 && sub == G % LPR;
            ns1 += acc ? (double)nv : 0.0;
            ns2 = acc ? fma((double)nv, (double)nv, ns2) : ns2;
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = l[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, l[u][h]);
      if (__any(mx > m[h] + kSlack)) {
        const float mn = wave_max_groups(fmaxf(mx, m[h]));
        const float sc = exp2_hw(m[h] - mn);
        m[h] = mn;
        Z[h] *= sc;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] *= sc;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float pu[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pu[h] = exp2_hw(l[u][h] - m[h]);
        Z[h] += pu[h];
      }
      // a masked row contributes p = 0; zeroing its V bits keeps a non-finite
      // value in the stand-in row from turning 0 * v into NaN
      const uint32_t vm = (st.j[u] >= 0) ? 0xFFFFFFFFu : 0u;
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const uint32_t w4[4] = {st.v[u][c].x & vm, st.v[u][c].y & vm, st.v[u][c].z & vm,
                                st.v[u][c].w & vm};
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const float v0 = bf_lo(w4[q2]), v1 = bf_hi(w4[q2]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][8 * c + 2 * q2] = fmaf(pu[h], v0, acc[h][8 * c + 2 * q2]);
            acc[h][8 * c + 2 * q2 + 1] = fmaf(pu[h], v1, acc[h][8 * c + 2 * q2 + 1]);
          }
        }
      }
    }
  };

  // Two stages in flight: the loads of one stage overlap the math of the other.
  constexpr int STEP = RPB * U;
  // The trip count is the same for every lane of the wave (lane groups past
  // the chunk's end consume masked rows), so the wave-wide maximum updates
  // in consume() see every lane and m stays wave-uniform.
  bool compact_run = false;
  if constexpr (COMPACT) {
    const int nfix = fl.ns + fl.nw;
    compact_run = p0 >= nfix;  // uniform over the workgroup
    if (compact_run) {
      // key ids of a compact stage, for the masks in consume()
      auto ids = [&](Stage &st, int base) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pp = base + u * RPB;
          st.j[u] = (pp < p1) ? s_idx[min(pp - p0, a.chunk - 1)] : -1;
        }
      };
      if (!spec_c || nfix != nfix_full) load_compact(sa, p0 + rg, nfix);
      ids(sa, p0 + rg);
      for (int base = p0; base < p1; base += 2 * STEP) {
        load_compact(sb, base + rg + STEP, nfix);
        ids(sb, base + rg + STEP);
        consume(sa);
        load_compact(sa, base + rg + 2 * STEP, nfix);
        ids(sa, base + rg + 2 * STEP);
        consume(sb);
      }
    }
  }
  // Evidence staging: write the block of rows [blk, blk + nr) out of LDS
  // (every thread of the workgroup takes part; barriers on both sides).
  // Prior from the statistics: each flushed block's prior weights into this
  // thread's fp64 sum.

  auto ev_flush = [&](int blk, int nr) {
    if constexpr (EV_LDS) {
      __syncthreads();
      float *lg = a.logits + (lrow * a.lld + blk) * G;
      for (int i = tid; i < nr * G; i += kThreads) lg[i] = s_evl[i];
      float *nm = a.key_norm + lrow * a.nld + blk;
      for (int i = tid; i < nr; i += kThreads) nm[i] = s_evn[i];
      if constexpr (STATS) {  // the block's prior weights, a few per thread
        float w = 0.f;
        for (int i = tid; i < nr; i += kThreads) w += prior_w(s_evn[i], blk + i, st_muf, st_cz, (float)(n - 1), st_ct);
        ns1 += (double)w;
      }
      __syncthreads();
    }
  };
  static_assert(!EV_LDS || kEvBlock % (2 * STEP) == 0, "a staging block is whole loop trips");
  static_assert(!EV_LDS || !COMPACT, "evidence mode streams the cache rows");
  if (!compact_run) {
    load_stage(sa, p0 + rg);
    for (int base = p0; base < p1; base += 2 * STEP) {
      load_stage(sb, base + rg + STEP);
      consume(sa);
      load_stage(sa, base + rg + 2 * STEP);
      consume(sb);
      if constexpr (EV_LDS) {
        // a block is complete, or the chunk ends inside this one
        const int next = base + 2 * STEP;
        if (((next - p0) & (kEvBlock - 1)) == 0 || next >= p1) {
          const int blk = p0 + ((base - p0) & ~(kEvBlock - 1));
          ev_flush(blk, min(next, p1) - blk);
        }
      }
    }
  }

  // Merge the lane groups of each wave as a reduce-scatter: in the round
  // with partner lane ^ off, each lane keeps half of its dimensions (the half
  // chosen by bit `off` of its lane id), receives the partner's values for
  // that half and combines them; the other half goes to the partner.  The
  // xor-8 round stays inside a 16-lane row and uses a DPP rotate.
  const int lane = tid & 63, wv = tid >> 6;
  int dim_off = 0;
  auto merge_round = [&](auto off_c, auto half_c) {
    constexpr int OFF = decltype(off_c)::value;
    constexpr int HALF = decltype(half_c)::value;
    const bool bit = (lane & OFF) != 0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (OFF == 8) {  // row_ror:8 == lane ^ 8 within a row (DPP)
        Z[h] += dpp_f32<0x128>(Z[h]);  // the reference m is wave-uniform: partials just add
#pragma unroll
        for (int i = 0; i < HALF; ++i) {
          const float keep = bit ? acc[h][HALF + i] : acc[h][i];
          const float send = bit ? acc[h][i] : acc[h][HALF + i];
          acc[h][i] = keep + dpp_f32<0x128>(send);
        }
      } else {  // lane halves: permlane swaps (same sums, same order of operands)
        Z[h] = xsum<OFF>(Z[h]);
#pragma unroll
        for (int i = 0; i < HALF; ++i) acc[h][i] = xsum_scatter<OFF>(acc[h][i], acc[h][HALF + i]);
      }
    }
    dim_off += bit ? HALF : 0;
  };
  if constexpr (LPR == 8) {
    merge_round(std::integral_constant<int, 8>{}, std::integral_constant<int, DPL / 2>{});
    merge_round(std::integral_constant<int, 16>{}, std::integral_constant<int, DPL / 4>{});
    merge_round(std::integral_constant<int, 32>{}, std::integral_constant<int, DPL / 8>{});
  } else {
    merge_round(std::integral_constant<int, 16>{}, std::integral_constant<int, DPL / 2>{});
    merge_round(std::integral_constant<int, 32>{}, std::integral_constant<int, DPL / 4>{});
  }
  constexpr int KEPT = (LPR == 8) ? DPL / 8 : DPL / 4;  // dims per lane after the rounds
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int i = 0; i < KEPT; ++i) {
      const int li = dim_off + i;  // index in the lane's slices
      s_acc[wv][h][slice(li / 8) + li % 8] = acc[h][i];
    }
    if (lane == 0) {
      s_m[wv][h] = m[h];
      s_z[wv][h] = Z[h];
    }
  }
  __shared__ double s_ns[NW][2];
  if constexpr (EVID) {
    if (STATS || a.nsum) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        ns1 += __shfl_xor(ns1, off);
        ns2 += __shfl_xor(ns2, off);
      }
      if (lane == 0) {
        s_ns[wv][0] = ns1;
        s_ns[wv][1] = ns2;
      }
    }
  }
  __syncthreads();
  if constexpr (EVID) {
    if (a.nsum && tid == 0) {
      double t1 = 0.0, t2 = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        t1 += s_ns[w][0];
        t2 += s_ns[w][1];
      }
      a.nsum[(lrow * a.stride + split) * 2 + 0] = t1;
      a.nsum[(lrow * a.stride + split) * 2 + 1] = t2;
    }
    if (STATS && tid == 0) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += s_ns[w][0];
      a.wpart[lrow * a.stride + split] = t;
    }
  }

  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, e = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float o = 0.f, z = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = exp2_hw(s_m[w][h] - M);
      o = fmaf(s_acc[w][h][e], sc, o);
      z = fmaf(s_z[w][h], sc, z);
    }
    const size_t slot = ((size_t)(a.pe ? zb : b) * a.Hq + g * G + h) * a.stride + split;
    a.part_o[slot * D + e] = o;
    if (e == 0) {
      a.part_ml[slot * 2 + 0] = M;
      a.part_ml[slot * 2 + 1] = z;
    }
  }
  append_store();
}

template <int D, int G, bool PAGED, int MODE, bool EVID, bool STATS = false>
__global__ __launch_bounds__(kThreads) void partial_kernel(PartialArgs a) {
  const PairBlock pb = a.wt.n > 0 ? table_block(a.wt, linear_block(), a.kv.Hkv)
                                  : pair_block(linear_block(), gridDim.x, gridDim.y, gridDim.z, MODE == MODE_FAST);
  partial_body<D, G, PAGED, MODE, EVID, false, STATS>(a, pb.blk, pb.h, pb.z);
}

// Fast step reading its selected rows from the compact copy.
template <int D, int G, bool PAGED>
__global__ __launch_bounds__(kThreads) void fast_compact_kernel(PartialArgs a) {
  const PairBlock pb = pair_block(linear_block(), gridDim.x, gridDim.y, gridDim.z);
  partial_body<D, G, PAGED, MODE_FAST, false, true>(a, pb.blk, pb.h, pb.z);
}

// Compact copy of the selected rows: row i of (sequence, kv head) holds the
// K and V rows of selection entry i.  D / 8 lanes move a row with 16-byte
// loads and stores; a workgroup moves kThreads * 8 / D rows.
template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void compact_kernel(PartialArgs a, uint16_t *ck, uint16_t *cv) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (b < 0) return;
  const int g = blockIdx.y;
  const int i = blockIdx.x * RPB + (int)threadIdx.x / LPR;
  const int sub = (int)threadIdx.x % LPR;
  const int hs = (a.sel_heads == 1) ? 0 : g;
  const int cnt = min(max(a.sel_count[b * a.sel_heads + hs], 0), a.sel_k);
  if (i >= cnt) return;
  const int n = clamp_len(a.seq_len, b, a.max_len);
  const int j = a.sel_idx[((size_t)b * a.sel_heads + hs) * a.sel_k + i];
  if (j < 0 || j >= n) return;
  const size_t src = kv_row<D, PAGED>(a.kv, b, g, j) + 8 * sub;
  const size_t dst = (((size_t)b * a.kv.Hkv + g) * a.sel_k + i) * D + 8 * sub;
  const uint4 kk = ldg16(a.kv.k + src), vv = ldg16(a.kv.v + src);
  *reinterpret_cast<uint4 *>(ck + dst) = kk;
  *reinterpret_cast<uint4 *>(cv + dst) = vv;
}

// Cache append: rows t < T of the new tokens of sequence batch_ids[z] go to
// cache rows seq_len[b] - T + t (rows below 0 are skipped).  One thread per
// 16-byte slice of a K and a V row; grid (slices / kThreads, batch entries).
template <int D, bool PAGED>
__global__ __launch_bounds__(kThreads) void append_kernel(KVView kv, const int32_t *seq_len,
                                                          const int32_t *batch_ids, int B, int max_len,
                                                          const uint16_t *k_new, const uint16_t *v_new,
                                                          int T) {
  constexpr int SPR = D / 8;  // 16-byte slices per row
  const int b = batch_seq(batch_ids, blockIdx.y, B);
  if (b < 0) return;
  const int i = blockIdx.x * kThreads + (int)threadIdx.x;
  if (i >= T * kv.Hkv * SPR) return;
  const int c = i % SPR, g = (i / SPR) % kv.Hkv, t = i / (SPR * kv.Hkv);
  const int j = clamp_len(seq_len, b, max_len) - T + t;
  if (j < 0) return;
  const size_t src = (((size_t)b * T + t) * kv.Hkv + g) * D + 8 * c;
  const size_t dst = kv_row<D, PAGED>(kv, b, g, j) + 8 * c;
  const uint4 kk = ldg16(k_new + src), vv = ldg16(v_new + src);
  *reinterpret_cast<uint4 *>(const_cast<uint16_t *>(kv.k) + dst) = kk;
  *reinterpret_cast<uint4 *>(const_cast<uint16_t *>(kv.v) + dst) = vv;
}

// Key-norm statistics of appended rows: one wave per (kv head, listed
// sequence) adds the norms of its T new K rows (rows j < 0 are skipped) in
// row order.
template <int D>
__global__ __launch_bounds__(64) void norm_add_kernel(double *nstat, const int32_t *seq_len,
                                                      const int32_t *batch_ids, int B, int Hkv, int max_len,
                                                      const uint16_t *k_new, int T) {
  const int b = batch_seq(batch_ids, blockIdx.y, B);
  if (b < 0) return;
  const int g = blockIdx.x, lane = threadIdx.x;
  const int n = clamp_len(seq_len, b, max_len);
  double s1 = 0.0, s2 = 0.0;
  for (int t = max(0, T - n); t < T; ++t) {
    const uint4 x = (lane < D / 8) ? ldg16(k_new + (((size_t)b * T + t) * Hkv + g) * D + 8 * lane)
                                   : make_uint4(0u, 0u, 0u, 0u);
    const float nu = wave_row_norm<D>(x);
    s1 += (double)nu;
    s2 = fma((double)nu, (double)nu, s2);
  }
  if (lane == 0) {
    nstat[((size_t)b * Hkv + g) * 2 + 0] += s1;
    nstat[((size_t)b * Hkv + g) * 2 + 1] += s2;
  }
}

// Slow (dense with evidence) and fast shares of one decode step in a single
// grid: linear blocks [0, ns) are the slow grid (s_splits x Hkv x slow
// sequences), the rest the fast grid.  The two sets of sequences are
// disjoint, so nothing orders one share after the other.  With PEND the grid
// ends with np workgroups of another layer's pending selection (its key
// pass, chunk-major over (chunk, head row, batch entry)): a selection that
// reads only that layer's buffers, so it shares the grid with this step.
// Placed last, its latency-bound workgroups start as the attention
// workgroups finish and fill the wave's tail (placed first, they took the
// attention's slots and serialised: workgroups of one kernel all get the
// attention's register allocation).
template <int D, int G, bool PAGED, bool PEND, bool STATS = false>
__global__ __launch_bounds__(kThreads) void copartial_kernel(PartialArgs s, PartialArgs f, int s_splits,
                                                             int f_splits, int Hkv, int ns,
                                                             SelectLaunch pend, int np) {
  int id = blockIdx.x;
  const int nt = gridDim.x - np;
  if constexpr (PEND) {
    if (id >= nt) {
      id -= nt;
      const PairBlock pb = pair_block(id, pend.ws.P, pend.H, pend.batch_n);
      keys_body<true>(pend, pb.blk, pb.h, pb.z);
      return;
    }
  }
  if (id < ns) {
    const PairBlock pb = s.wt.n > 0 ? table_block(s.wt, id, Hkv)
                                    : pair_block(id, s_splits, Hkv, ns / (s_splits * Hkv), false);
    partial_body<D, G, PAGED, MODE_SLOW, true, false, STATS>(s, pb.blk, pb.h, pb.z);
  } else {
    id -= ns;
    const PairBlock pb = f.wt.n > 0 ? table_block(f.wt, id, Hkv)
                                    : pair_block(id, f_splits, Hkv, (nt - ns) / (f_splits * Hkv));
    partial_body<D, G, PAGED, MODE_FAST, false>(f, pb.blk, pb.h, pb.z);
  }
}

struct FinalArgs {
  int B, max_len;
  const int32_t *seq_len;
  const int32_t *batch_ids;
  int Hq, Hkv;
  int chunk, stride;
  int splits;  // planned splits per (sequence, kv head); unused ones hold Z = 0
  const float *part_o;
  const float *part_ml;
  float *out;
  const float *logits;
  int lld;
  float *evidence;
  int ld;
  const int32_t *sel_idx;
  const int32_t *sel_count;
  int sel_heads, sel_k, n_sink, window;
  // selector prior (evidence blocks; null nsum: not computed)
  const double *nsum;
  const float *key_norm;
  float norm_coef, pos_tau;
  double *sel_wsum;
  SelRowMeta *sel_meta;
  uint32_t *sel_ghist;
  int selP;
  int pe;  // 1: partial buffers indexed by batch entry instead of sequence id
  // Key-norm statistics [B*Hkv][2], stored by the evidence blocks of a step
  // that forms the prior (null: none kept): the sums of this pass, or with
  // keys the partial kernel's updated statistics nnext
  double *nstat;
  // Prior formed from the statistics by the partial kernel (keys = 1, nsum
  // null): the evidence blocks also run the selection's key pass (sel) on
  // the fused scores, from the splits' prior-weight sums wpart and the row
  // constants the partial kernel wrote to sel_meta.
  int keys;
  const double *wpart;
  const double *nnext;
  SelectLaunch sel;
  WorkTable wt;  // per-entry split counts of the partial grid (wt.n = 0: splits)
};

// Merge (m2, z2) into the running softmax pair (m, z): both are a log2-domain
// reference and the sum of 2^(l - reference) over their keys.
__device__ __forceinline__ void mz_merge(float &m, float &z, float m2, float z2) {
  const float mn = fmaxf(m, m2);
  z = z * exp2_hw(m - mn) + z2 * exp2_hw(m2 - mn);
  m = mn;
}

// grid.x = G combine blocks (one per query head of the group) followed, for
// slow steps with evidence, by one block per kEvidChunk keys.  Every block
// issues all of its global loads before it needs the merged maxima, so a
// block costs one memory round trip.  KEYS: the evidence blocks also run
// the selection's key pass (FinalArgs::keys).
template <int D, int G, int MODE, bool EVID, bool KEYS = false>
__device__ __forceinline__ void finalize_body(const FinalArgs &a, int x, int g, int zb) {
  constexpr int NW = kThreads / 64;

  const int b = batch_seq(a.batch_ids, zb, a.B);
  if (b < 0) return;
  const bool comb = x < G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t hbase = (size_t)b * a.Hq + (size_t)g * G;
  const size_t pbase = (size_t)(a.pe ? zb : b) * a.Hq + (size_t)g * G;  // rows of the partial buffers

  if (comb) {
    // every planned split of the entry: those past the row list wrote Z = 0
    // and are skipped, so no length is read before the partials
    const int S = entry_splits(a.wt, zb, a.splits);
    // PARTS groups of D/4 threads; group `part` merges partials part,
    // part + PARTS, ... (four at a time, their loads in flight together)
    // into a running (m, z, o); the groups are then merged through LDS.
    constexpr int TPP = D / 4;
    constexpr int PARTS = kThreads / TPP;
    const size_t row = hbase + x, prow = pbase + x;
    const int e4 = tid % TPP, part = tid / TPP;
    const float *pm = a.part_ml + prow * a.stride * 2;
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o + prow * a.stride * D) + e4;
    float m = kNegBig, z = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = part; s0 < S; s0 += 4 * PARTS) {
      float4 v[4];
      float ms[4], zs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = min(s0 + i * PARTS, S - 1);
        v[i] = po[(size_t)s * TPP];
        ms[i] = pm[s * 2];
        zs[i] = pm[s * 2 + 1];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (s0 + i * PARTS < S && zs[i] > 0.f) {
          const float mn = fmaxf(m, ms[i]);
          const float c = exp2_hw(m - mn), w = exp2_hw(ms[i] - mn);
          z = z * c + zs[i] * w;
          o.x = o.x * c + v[i].x * w;
          o.y = o.y * c + v[i].y * w;
          o.z = o.z * c + v[i].z * w;
          o.w = o.w * c + v[i].w * w;
          m = mn;
        }
      }
    }
    __shared__ float s_pm[PARTS], s_pz[PARTS];
    __shared__ float4 s_po[PARTS][TPP];
    if (e4 == 0) {
      s_pm[part] = m;
      s_pz[part] = z;
    }
    s_po[part][e4] = o;
    __syncthreads();
    if (part == 0) {
      float M = s_pm[0];
#pragma unroll
      for (int p = 1; p < PARTS; ++p) M = fmaxf(M, s_pm[p]);
      float Z = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int p = 0; p < PARTS; ++p) {
        const float w = exp2_hw(s_pm[p] - M);
        const float4 t = s_po[p][e4];
        Z = fmaf(s_pz[p], w, Z);
        acc.x = fmaf(t.x, w, acc.x);
        acc.y = fmaf(t.y, w, acc.y);
        acc.z = fmaf(t.z, w, acc.z);
        acc.w = fmaf(t.w, w, acc.w);
      }
      const float rz = (Z > 0.f) ? 1.0f / Z : 0.f;
      reinterpret_cast<float4 *>(a.out + row * D)[e4] =
          make_float4(acc.x * rz, acc.y * rz, acc.z * rz, acc.w * rz);
    }
    return;
  }

  if constexpr (EVID) {
    const int n = clamp_len(a.seq_len, b, a.max_len);
    if ((x - G) * kEvidChunk >= n) return;
    // the splits holding the row's keys, never past the entry's planned
    // splits (a host row-count hint below n leaves keys unplanned)
    const int S = min((n + a.chunk - 1) / a.chunk, entry_splits(a.wt, zb, a.splits));
    const size_t lrow = (size_t)b * a.Hkv + g;
    const int j0 = (x - G) * kEvidChunk;
    const int j1 = min(n, j0 + kEvidChunk);
    constexpr int PER = kEvidChunk / kThreads;
    // Every global load of the block goes out before the first use: the
    // chunk's logits (one 16-byte load per key and 4 heads) and key norms,
    // the partials' (max, sum) pairs and, for the selector's prior, the
    // per-split key-norm sums.
    const bool prior = KEYS || a.nsum != nullptr;
    float lg[PER][G], nv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = j0 + tid + i * kThreads;
      const float *lp = a.logits + (lrow * a.lld + (size_t)min(j, j1 - 1)) * G;
      if constexpr (G % 4 == 0) {
#pragma unroll
        for (int c = 0; c < G / 4; ++c) {
          const float4 t = reinterpret_cast<const float4 *>(lp)[c];
          lg[i][4 * c + 0] = t.x; lg[i][4 * c + 1] = t.y; lg[i][4 * c + 2] = t.z; lg[i][4 * c + 3] = t.w;
        }
      } else if constexpr (G == 2) {
        const float2 t = *reinterpret_cast<const float2 *>(lp);
        lg[i][0] = t.x; lg[i][1] = t.y;
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) lg[i][h] = lp[h];
      }
      nv[i] = prior ? a.key_norm[lrow * a.ld + min(j, j1 - 1)] : 0.f;
    }
    // the key pass's histogram is cleared while the loads are in flight
    // (the merge's barrier below orders it before the pass)
    __shared__ std::conditional_t<KEYS, KeysLds, int> s_keys;
    if constexpr (KEYS) keys_clear(s_keys);
    // merged (max, sum) of every head of the group over the S partials, and
    // the row's key-norm sums (fixed order; every chunk block repeats them)
    float m[G], z[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegBig;
      z[h] = 0.f;
    }
    double s1 = 0.0, s2 = 0.0, sw = 0.0;
    float rm_muf = 0.f, rm_cz = 0.f;
    if constexpr (KEYS) {
      const SelRowMeta rm = a.sel_meta[lrow];
      rm_muf = rm.muf;
      rm_cz = rm.cz;
    }
    for (int s = tid; s < S; s += kThreads) {
      float ml[G][2];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float *ml2 = a.part_ml + ((pbase + h) * a.stride + s) * 2;
        ml[h][0] = ml2[0];
        ml[h][1] = ml2[1];
      }
      double n1 = 0.0, n2 = 0.0, w1 = 0.0;
      if constexpr (KEYS) {
        w1 = a.wpart[lrow * a.stride + s];
      } else if (prior) {
        n1 = a.nsum[(lrow * a.stride + s) * 2 + 0];
        n2 = a.nsum[(lrow * a.stride + s) * 2 + 1];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) mz_merge(m[h], z[h], ml[h][0], ml[h][1]);
      s1 += n1;
      s2 += n2;
      sw += w1;
    }
    __shared__ float s_m[NW][G], s_z[NW][G];
    __shared__ double s_d[NW][3], s_w[NW];
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m[h], off), z2 = __shfl_xor(z[h], off);
        mz_merge(m[h], z[h], m2, z2);
      }
      if (lane == 0) {
        s_m[wv][h] = m[h];
        s_z[wv][h] = z[h];
      }
    }
    if (prior) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        s1 += __shfl_xor(s1, off);
        s2 += __shfl_xor(s2, off);
        sw += __shfl_xor(sw, off);
      }
      if (lane == 0) {
        s_d[wv][0] = s1;
        s_d[wv][1] = s2;
        s_d[wv][2] = sw;
      }
    }
    __syncthreads();
    float M[G], rz[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mm = s_m[0][h], zz = s_z[0][h];
#pragma unroll
      for (int w = 1; w < NW; ++w) mz_merge(mm, zz, s_m[w][h], s_z[w][h]);
      M[h] = mm;
      rz[h] = 1.0f / ((float)G * zz);
    }
    float fv[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = j0 + tid + i * kThreads;
      float f = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) f = fmaf(exp2_hw(lg[i][h] - M[h]), rz[h], f);
      fv[i] = f;
      if (j < j1) a.evidence[lrow * a.ld + j] = f;
    }
    if (!prior) return;
    // The selector's prior for this 2048-key chunk (the selector's chunk p):
    // mean and population std of the row's key norms, then the chunk's sum
    // of prior weights.  Chunk 0 also stores the row constants, and the
    // blocks clear the row's bucket histogram between them, so the selection
    // can start at its key pass.
    const int pch = x - G;
    s1 = 0.0;
    s2 = 0.0;
    sw = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      s1 += s_d[w][0];
      s2 += s_d[w][1];
      sw += s_d[w][2];
    }
    // the row's key-norm statistics: exact from this pass, or those the
    // partial kernel formed the prior from
    if (a.nstat != nullptr && pch == 0 && tid == 0) {
      a.nstat[lrow * 2 + 0] = KEYS ? a.nnext[lrow * 2 + 0] : s1;
      a.nstat[lrow * 2 + 1] = KEYS ? a.nnext[lrow * 2 + 1] : s2;
    }
    if constexpr (KEYS) {
      // the selection's key pass on this chunk (the selector's chunk pch):
      // s = (1 - lambda) f + lambda w / W with the partial kernel's row
      // constants and weight sums, so w is the weight it summed, bit for bit
      static_assert(kEvidChunk == kSelChunk && PER == kPT, "evidence blocks are selector chunks");
      RowGeo r;
      row_geo_n(a.sel, b, g, n, r);
      const float cf = 1.0f - a.sel.lambda;
      const float cr = sw > 0.0 ? (float)((double)a.sel.lambda / sw) : 0.f;
      const float ct = kLog2e / a.pos_tau;
      const float tq = (float)(n - 1);
      float sc[PER];
      int jj[PER];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int j = j0 + tid + i * kThreads;
        const float w = (j < j1) ? prior_w(nv[i], j, rm_muf, rm_cz, tq, ct) : 0.f;
        sc[i] = fmaf(cf, fv[i], cr * w);
        jj[i] = j;
      }
      if (a.sel.fused_out) {
        float *fo = a.sel.fused_out + r.row * a.sel.fo_ld;
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (jj[i] < j1) fo[jj[i]] = sc[i];
      }
      if (pch >= r.nch) return;  // no candidates in this chunk
      keys_core(a.sel, r, pch, sc, jj, s_keys);
      return;
    }
    float muf, cz;
    prior_consts(s1, s2, n, a.norm_coef, &muf, &cz);
    const float ct = kLog2e / a.pos_tau;
    const float tq = (float)(n - 1);
    float wc = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = j0 + tid + i * kThreads;
      wc += (j < j1) ? prior_w(nv[i], j, muf, cz, tq, ct) : 0.f;
    }
    double W = (double)wc;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) W += __shfl_xor(W, off);
    if (lane == 0) s_w[wv] = W;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) t += s_w[w];
      a.sel_wsum[lrow * a.selP + pch] = t;
      if (pch == 0) {
        a.sel_meta[lrow].muf = muf;
        a.sel_meta[lrow].cz = cz;
      }
    }
    const int nch = (n + kEvidChunk - 1) / kEvidChunk;
    for (int i = pch * kThreads + tid; i < 4096; i += nch * kThreads) a.sel_ghist[lrow * 4096 + i] = 0u;
  }
}

template <int D, int G, int MODE, bool EVID, bool KEYS = false>
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalArgs a) {
  const PairBlock pb = pair_block(linear_block(), gridDim.x, gridDim.y, gridDim.z);
  finalize_body<D, G, MODE, EVID, KEYS>(a, pb.blk, pb.h, pb.z);
}

// Slow and fast finalize blocks of one decode step in a single grid: the
// slow pairs' evidence blocks, their combine blocks, then the fast combine
// blocks (G x Hkv x fast sequences); with PEND it ends with the pending
// selection's pick pass; with KEYS the slow share's evidence blocks run its
// own selection's key pass.
template <int D, int G, bool PEND, bool KEYS = false>
__global__ __launch_bounds__(kThreads) void cofinal_kernel(FinalArgs s, FinalArgs f, int s_gx, int f_gx,
                                                           int Hkv, int ns, SelectLaunch pend, int np) {
  int id = blockIdx.x;
  const int nt = gridDim.x - np;
  if constexpr (PEND) {
    if (id >= nt) {
      id -= nt;
      const PairBlock pb = pair_block(id, pend.ws.P, pend.H, pend.batch_n);
      pick_body(pend, pb.blk, pb.h, pb.z);
      return;
    }
  }
  if (id < ns) {
    // the evidence blocks (the longest) are dispatched first
    const int ne = s_gx - G, pairs = ns / s_gx;
    if (id < ne * pairs) {
      const PairBlock pb = pair_block(id, ne, Hkv, pairs / Hkv);
      finalize_body<D, G, MODE_SLOW, true, KEYS>(s, G + pb.blk, pb.h, pb.z);
    } else {
      id -= ne * pairs;
      const PairBlock pb = pair_block(id, G, Hkv, pairs / Hkv);
      finalize_body<D, G, MODE_SLOW, true, KEYS>(s, pb.blk, pb.h, pb.z);
    }
  } else {
    id -= ns;
    const PairBlock pb = pair_block(id, f_gx, Hkv, (nt - ns) / (f_gx * Hkv));
    finalize_body<D, G, MODE_FAST, false>(f, pb.blk, pb.h, pb.z);
  }
}

// Resident workgroups of one kernel across the device, cached per kernel and
// device (the kernel is a template argument so every instantiation keeps its
// own cache: all partial kernels share one function-pointer type).
template <auto KERN>
int resident_slots() {
  static int slots[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (slots[dev] == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, KERN, kThreads, 0) != hipSuccess || nb < 1) nb = 1;
    slots[dev] = nb * device_cu_count() * SFI_WAVES_OF_WG;
  }
  return slots[dev];
}

template <int D>
PartialArgs partial_args(const AttnLaunch &a) {
  PartialArgs p{};
  p.B = a.B; p.max_len = a.max_len;
  p.kv = a.kv; p.seq_len = a.seq_len; p.batch_ids = a.batch_ids; p.q = a.q; p.Hq = a.Hq;
  p.chunk = a.plan.chunk; p.stride = a.plan.stride; p.part_o = a.part_o; p.part_ml = a.part_ml;
  p.logits = a.logits; p.lld = a.lld; p.key_norm = a.key_norm; p.ld = a.ld; p.nld = a.nld;
  p.sel_idx = a.sel_idx; p.sel_count = a.sel_count; p.sel_heads = a.sel_heads; p.sel_k = a.sel_k;
  p.n_sink = a.n_sink; p.window = a.window;
  p.qscale = kLog2e / sqrtf((float)D);
  p.nsum = a.nsum;
  p.wpart = a.wpart;
  p.nnext = a.nnext;
  p.sel_meta = a.sel_meta;
  p.sel_ghist = a.sel_ghist;
  p.nsp = a.plan.splits;
  p.wt = a.wt;
  p.norm_coef = a.norm_coef;
  p.pos_tau = a.pos_tau;
  p.ck = a.ck;
  p.cv = a.cv;
  p.pe = a.part_by_entry ? 1 : 0;
  return p;
}

FinalArgs final_args(const AttnLaunch &a) {
  FinalArgs f{};
  f.B = a.B; f.max_len = a.max_len;
  f.seq_len = a.seq_len; f.batch_ids = a.batch_ids; f.Hq = a.Hq; f.Hkv = a.Hkv;
  f.chunk = a.plan.chunk; f.stride = a.plan.stride; f.splits = a.plan.splits;
  f.part_o = a.part_o; f.part_ml = a.part_ml;
  f.out = a.out; f.logits = a.logits; f.lld = a.lld; f.evidence = a.evidence; f.ld = a.ld;
  f.sel_idx = a.sel_idx; f.sel_count = a.sel_count; f.sel_heads = a.sel_heads;
  f.sel_k = a.sel_k; f.n_sink = a.n_sink; f.window = a.window;
  f.nsum = a.nsum; f.key_norm = a.key_norm; f.norm_coef = a.norm_coef; f.pos_tau = a.pos_tau;
  f.sel_wsum = a.sel_wsum; f.sel_meta = a.sel_meta; f.sel_ghist = a.sel_ghist; f.selP = a.selP;
  f.pe = a.part_by_entry ? 1 : 0;
  f.wt = a.wt;
  f.nstat = (a.nsum != nullptr || a.stats) ? a.kv.nstat : nullptr;
  if (a.stats && a.keysel != nullptr) {
    f.keys = 1;
    f.wpart = a.wpart;
    f.nnext = a.nnext;
    f.sel = *a.keysel;
  }
  return f;
}

// Longest row list of a fast step.
long long fast_rows(const AttnLaunch &a) {
  return (long long)std::min(a.n_sink, a.max_len) + std::min(a.window, a.max_len) + a.sel_k;
}

// Planning from host-known per-entry row counts (AttnLaunch::len_host).
bool hinted(const AttnLaunch &a) { return a.len_host != nullptr && a.batch_n > 0; }

long long host_max(const AttnLaunch &a) {
  long long m = 1;
  for (int z = 0; z < a.batch_n; ++z) m = std::max<long long>(m, a.len_host[z]);
  return m;
}

// A table pays where the entries' row counts differ: at least a tenth of a
// max-length plan's blocks would find no rows.  Entries of (nearly) one
// length keep the grid of the plain plan, sized from the longest hint,
// since a table costs each block a round trip for the prefix sums before
// its first row load.
bool tabled(const AttnLaunch &a) {
  if (!hinted(a) || a.batch_n > kMaxListed) return false;
  long long sum = 0;
  for (int z = 0; z < a.batch_n; ++z) sum += std::max(a.len_host[z], 0);
  return sum * 10 < 9LL * a.batch_n * host_max(a);
}

// Rows that size the plain plan: the longest hint, else the host bound.
long long plan_rows_of(const AttnLaunch &a, long long bound) {
  return hinted(a) ? std::min(bound, host_max(a)) : bound;
}

// Chunk for about R rows per block: a multiple of the granule, at most
// max_chunk, and at least what keeps every entry within the stride.
long long table_chunk(const AttnLaunch &a, long long R, int max_chunk) {
  const long long lmax = host_max(a);
  long long c = std::max(R, (lmax + a.plan.stride - 1) / a.plan.stride);
  c = (c + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
  return std::max<long long>(kSplitGranule, std::min<long long>(c, max_chunk));
}

// Splits of every entry at this chunk (at least one, so that an entry with
// no rows still writes its neutral partials and takes its fused append);
// the table in a.wt, the total number of entry-splits returned (-1 when it
// does not fit the 16-bit table).
long long fill_table(AttnLaunch &a, long long chunk) {
  long long acc = 0;
  a.wt.n = a.batch_n;
  a.wt.cum[0] = 0;
  int smax = 1;
  for (int z = 0; z < a.batch_n; ++z) {
    const long long L = std::max<long long>(a.len_host[z], 0);
    const long long c = std::max<long long>(1, (L + chunk - 1) / chunk);
    if (c > a.plan.stride) return -1;  // more splits than the partials hold
    smax = std::max<int>(smax, (int)c);
    acc += c;
    if (acc > 65535) return -1;
    a.wt.cum[z + 1] = (uint16_t)acc;
  }
  a.plan.chunk = (int)chunk;
  a.plan.splits = smax;
  return acc;
}

// Entry-splits of the table at this chunk, without filling it.
long long table_total(const AttnLaunch &a, long long chunk) {
  long long acc = 0;
  for (int z = 0; z < a.batch_n; ++z)
    acc += std::max<long long>(1, (std::max<long long>(a.len_host[z], 0) + chunk - 1) / chunk);
  return acc;
}

// One share alone: the smallest chunk of at least min_chunk rows whose
// blocks fit one wave of resident blocks, at most max_chunk rows per block
// (more waves past that).
bool plan_table(AttnLaunch &a, int slots, int min_chunk, int max_chunk) {
  long long lo = (std::max(min_chunk, kSplitGranule) + kSplitGranule - 1) / kSplitGranule;
  long long hi = std::max<long long>(lo, max_chunk / kSplitGranule);  // in granules; hi is taken if none fits
  while (lo < hi) {
    const long long mid = (lo + hi) / 2;
    if (table_total(a, table_chunk(a, mid * kSplitGranule, max_chunk)) * a.Hkv <= slots) hi = mid;
    else lo = mid + 1;
  }
  if (fill_table(a, table_chunk(a, lo * kSplitGranule, max_chunk)) < 0) {
    a.wt.n = 0;
    return false;
  }
  return true;
}

// Finalize blocks per (sequence, kv head) of a slow step: G combine blocks,
// then one evidence block per kEvidChunk keys.
int slow_final_blocks(const AttnLaunch &a, int G) {
  const int kv_max = a.plan.splits * a.plan.chunk;
  return G + (a.evidence ? (kv_max + kEvidChunk - 1) / kEvidChunk : 0);
}

template <int D, int G, bool PAGED>
hipError_t slow_t(const AttnLaunch &a_in, hipStream_t st) {
  AttnLaunch a = a_in;
  const bool side = a.evidence != nullptr || a.key_norm != nullptr;
  {
    // planned with the contiguous-cache kernel's occupancy, so a paged cache
    // gets the same split plan and therefore the same bits
    const int slots = side ? resident_slots<partial_kernel<D, G, false, MODE_SLOW, true>>()
                           : resident_slots<partial_kernel<D, G, false, MODE_SLOW, false>>();
    a.wt.n = 0;
    if (!(tabled(a) && plan_table(a, slots, kSplitGranule, kMaxSlowChunk)))
      a.plan = plan_splits(plan_rows_of(a, a.max_len), a.batch_n * a.Hkv, slots, a.plan.stride, kMaxSlowChunk, true);
  }
  const PartialArgs p = partial_args<D>(a);
  const dim3 grid = a.wt.n > 0 ? dim3((unsigned)a.wt.cum[a.wt.n] * a.Hkv) : dim3(a.plan.splits, a.Hkv, a.batch_n);
  if (a.stats && (!a.evidence || !a.keysel || a.nsum)) return hipErrorInvalidValue;
  if (a.stats)
    hipLaunchKernelGGL((partial_kernel<D, G, PAGED, MODE_SLOW, true, true>), grid, dim3(kThreads), 0, st, p);
  else if (side)
    hipLaunchKernelGGL((partial_kernel<D, G, PAGED, MODE_SLOW, true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((partial_kernel<D, G, PAGED, MODE_SLOW, false>), grid, dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  const FinalArgs f = final_args(a);
  dim3 g2(slow_final_blocks(a, G), a.Hkv, a.batch_n);
  if (a.evidence && f.keys)
    hipLaunchKernelGGL((finalize_kernel<D, G, MODE_SLOW, true, true>), g2, dim3(kThreads), 0, st, f);
  else if (a.evidence)
    hipLaunchKernelGGL((finalize_kernel<D, G, MODE_SLOW, true>), g2, dim3(kThreads), 0, st, f);
  else
    hipLaunchKernelGGL((finalize_kernel<D, G, MODE_SLOW, false>), g2, dim3(kThreads), 0, st, f);
  return hipGetLastError();
}

// Split plan of a fast step (chunks of the row list per (sequence, kv head)).
template <int D, int G>
SplitPlan fast_plan_t(const AttnLaunch &a) {
  const int slots = resident_slots<partial_kernel<D, G, false, MODE_FAST, false>>();
  return plan_splits(plan_rows_of(a, fast_rows(a)), a.batch_n * a.Hkv, slots, a.plan.stride, kMaxFastChunk, false);
}

template <int D, int G, bool PAGED>
hipError_t fast_t(const AttnLaunch &a_in, hipStream_t st) {
  AttnLaunch a = a_in;
  a.wt.n = 0;
  if (!a.planned) {
    const int slots = resident_slots<partial_kernel<D, G, false, MODE_FAST, false>>();
    if (!(tabled(a) && plan_table(a, slots, kSplitGranule, kMaxFastChunk))) a.plan = fast_plan_t<D, G>(a);
  }
  const PartialArgs p = partial_args<D>(a);
  const dim3 grid = a.wt.n > 0 ? dim3((unsigned)a.wt.cum[a.wt.n] * a.Hkv) : dim3(a.plan.splits, a.Hkv, a.batch_n);
  hipLaunchKernelGGL((partial_kernel<D, G, PAGED, MODE_FAST, false>), grid, dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const FinalArgs f = final_args(a);
  dim3 g2(G, a.Hkv, a.batch_n);
  hipLaunchKernelGGL((finalize_kernel<D, G, MODE_FAST, false>), g2, dim3(kThreads), 0, st, f);
  return hipGetLastError();
}

template <int D, int G, bool PAGED>
hipError_t fast_compact_t(const AttnLaunch &a_in, hipStream_t st) {
  AttnLaunch a = a_in;
  {
    // the index-gather kernel's plan, so both routes give the same bits
    const int slots = resident_slots<partial_kernel<D, G, false, MODE_FAST, false>>();
    a.plan = plan_splits(fast_rows(a), a.batch_n * a.Hkv, slots, a.plan.stride, kMaxFastChunk, false);
  }
  const PartialArgs p = partial_args<D>(a);
  dim3 grid(a.plan.splits, a.Hkv, a.batch_n);
  hipLaunchKernelGGL((fast_compact_kernel<D, G, PAGED>), grid, dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const FinalArgs f = final_args(a);
  dim3 g2(G, a.Hkv, a.batch_n);
  hipLaunchKernelGGL((finalize_kernel<D, G, MODE_FAST, false>), g2, dim3(kThreads), 0, st, f);
  return hipGetLastError();
}

template <int D, bool PAGED>
hipError_t compact_t(const AttnLaunch &a, uint16_t *ck, uint16_t *cv, hipStream_t st) {
  const PartialArgs p = partial_args<D>(a);
  constexpr int RPB = kThreads / (D / 8);
  dim3 grid((a.sel_k + RPB - 1) / RPB, a.Hkv, a.batch_n);
  hipLaunchKernelGGL((compact_kernel<D, PAGED>), grid, dim3(kThreads), 0, st, p, ck, cv);
  return hipGetLastError();
}

// A slow step (with evidence) for one set of sequences and a fast step for
// another, co-launched: one partial grid and one finalize grid.  Both shares
// are planned with the same number of rows per workgroup, so the workgroups
// of the combined grid carry about equal bytes and the grid fills the
// resident slots about once.
// The co-launched kernels take both shares' arguments (and a pending
// selection's) by value: within the 4 KB kernel-argument segment.
static_assert(2 * sizeof(PartialArgs) + sizeof(SelectLaunch) + 64 <= 4096, "copartial arguments");
static_assert(2 * sizeof(FinalArgs) + sizeof(SelectLaunch) + 64 <= 4096, "cofinal arguments");

// Both shares of a co-launched step planned from their entries' row counts:
// the k-wave search of the max_len plan below with the exact block count of
// each R (a table entry per listed entry, none past its rows).  False when
// a table does not fit.
bool plan_step_tables(AttnLaunch &sa, AttnLaunch &fa, int slots) {
  sa.wt.cum[0] = fa.wt.cum[0] = 0;
  // one share: the plan of its own launcher (the same chunks, the same bits)
  if (fa.batch_n == 0) {
    fa.plan = SplitPlan{1, 0, fa.plan.stride};
    return plan_table(sa, slots, kSplitGranule, kMaxSlowChunk);
  }
  if (sa.batch_n == 0) {
    sa.plan = SplitPlan{1, 0, sa.plan.stride};
    return plan_table(fa, slots, kSplitGranule, kMaxFastChunk);
  }
  const long long Ls = host_max(sa), Lf = host_max(fa);
  long long smin = kSplitGranule;  // fewest rows per slow block
  auto chunk_s = [&](long long R) { return table_chunk(sa, std::max(R, smin), kMaxSlowChunk); };
  auto chunk_f = [&](long long R) { return table_chunk(fa, std::max<long long>(R, kMinFastTableChunk), kMaxFastChunk); };
  auto blocks_at = [&](long long R) {
    return table_total(sa, chunk_s(R)) * sa.Hkv + table_total(fa, chunk_f(R)) * fa.Hkv;
  };
  auto rows_per_wg = [&](long long R) { return std::max(std::min(chunk_s(R), Ls), std::min(chunk_f(R), Lf)); };
  const long long Rmax = (std::max(Ls, Lf) + kSplitGranule - 1) / kSplitGranule;  // in granules
  long long best_cost = -1, best_R = Rmax;
  int best_k = 0;
  // a fast block never holds fewer rows than this, so no plan of k waves
  // costs less than k x (floor + block cost): the search stops there
  const long long floor_rows = std::min<long long>(kMinFastTableChunk, Lf);
  auto search = [&]() {
    best_cost = -1;
    best_R = Rmax;
    best_k = 0;
    bool fits = false;
    long long hi0 = Rmax;  // fits every k from the first that fits on
    for (int k = 1; k <= 16; ++k) {
      if (best_cost >= 0 && k * (floor_rows + kPlanBlockCost) >= best_cost) break;
      const long long cap = (long long)k * slots;
      if (!fits) {
        if (blocks_at(Rmax * kSplitGranule) > cap) continue;
        fits = true;
      }
      long long lo = 1, hi = hi0;  // hi fits
      while (lo < hi) {
        const long long mid = (lo + hi) / 2;
        if (blocks_at(mid * kSplitGranule) <= cap) hi = mid;
        else lo = mid + 1;
      }
      hi0 = hi;
      const long long cost = k * (rows_per_wg(hi * kSplitGranule) + kPlanBlockCost);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best_R = hi;
        best_k = k;
      }
    }
  };
  search();
  // Several waves: the dispatcher refills freed slots, so slow blocks may be
  // longer than the fast ones; fewer slow blocks pay fewer prologues and
  // evidence flushes (at the ragged batch 2048-row slow blocks took the
  // co-launched step from 164-166 to 158-159 us; in a one-wave plan they
  // would leave the slow share too few blocks).
  if (best_k > 1) {
    smin = kMultiWaveSlowChunk;
    search();
  }
  const long long R = best_cost < 0 ? kMaxFastChunk : best_R * kSplitGranule;
  if (fill_table(sa, chunk_s(R)) < 0) {
    sa.wt.n = 0;
    return false;
  }
  if (fill_table(fa, chunk_f(R)) < 0) {
    sa.wt.n = fa.wt.n = 0;
    return false;
  }
  if ((long long)sa.wt.cum[sa.wt.n] * sa.Hkv + (long long)fa.wt.cum[fa.wt.n] * fa.Hkv > 0x7fffffffLL) {
    sa.wt.n = fa.wt.n = 0;
    return false;
  }
  return true;
}

template <int D, int G, bool PAGED>
hipError_t step_t(const AttnLaunch &sa_in, const AttnLaunch &fa_in, hipStream_t st,
                  const SelectLaunch *pend) {
  AttnLaunch sa = sa_in, fa = fa_in;
  const int slots = resident_slots<copartial_kernel<D, G, false, false>>();
  sa.wt.n = 0;
  fa.wt.n = 0;
  // tables for both shares when both carry hints and either is ragged
  const bool tab = (sa.batch_n == 0 || (hinted(sa) && sa.batch_n <= kMaxListed)) &&
                   (fa.batch_n == 0 || (hinted(fa) && fa.batch_n <= kMaxListed)) && (tabled(sa) || tabled(fa));
  if (tab && plan_step_tables(sa, fa, slots)) {
    // planned from the entries' own row counts
  } else if (sa.batch_n == 0) {  // fast share only (a step that carries a pending selection)
    fa.plan = plan_splits(plan_rows_of(fa, fast_rows(fa)), fa.batch_n * fa.Hkv, slots, fa.plan.stride,
                          kMaxFastChunk, false);
    sa.plan = SplitPlan{1, 0, sa.plan.stride};
  } else if (fa.batch_n == 0) {  // slow share only
    sa.plan = plan_splits(plan_rows_of(sa, sa.max_len), sa.batch_n * sa.Hkv, slots, sa.plan.stride,
                          kMaxSlowChunk, true);
    fa.plan = SplitPlan{1, 0, fa.plan.stride};
  } else {
    const long long Ls = plan_rows_of(sa, sa.max_len), Lf = plan_rows_of(fa, fast_rows(fa));
    const long long ps = (long long)sa.batch_n * sa.Hkv, pf = (long long)fa.batch_n * fa.Hkv;
    const int s_stride = sa.plan.stride, f_stride = fa.plan.stride;
    // workgroups of the combined grid at R rows per workgroup (non-increasing in R)
    auto plan_at = [&](long long R) {
      sa.plan = plan_rows(Ls, s_stride, R, kMaxSlowChunk);
      fa.plan = plan_rows(Lf, f_stride, R, kMaxFastChunk);
      return ps * sa.plan.splits + pf * fa.plan.splits;
    };
    auto rows_per_wg = [&]() {
      return std::max(std::min<long long>(sa.plan.chunk, Ls), std::min<long long>(fa.plan.chunk, Lf));
    };
    // For k waves of resident workgroups take the smallest R (a multiple of
    // the granule) whose grid fits k waves, and keep the k whose makespan
    // estimate, k x the largest rows per workgroup, is least.  One wave is
    // best when it fits without starving one share (a second wave doubles
    // the runtime); the fast share's chunk is capped (its row ids are staged
    // in LDS), so a large fast share can need several waves, and a one-wave
    // plan could then leave each slow workgroup a whole sequence.
    const long long Rmax = (std::max(Ls, Lf) + kSplitGranule - 1) / kSplitGranule;  // in granules
    long long best_cost = -1, best_R = Rmax;
    for (int k = 1; k <= 16; ++k) {
      const long long cap = (long long)k * slots;
      if (plan_at(Rmax * kSplitGranule) > cap) continue;
      long long lo = 1, hi = Rmax;  // hi fits
      while (lo < hi) {
        const long long mid = (lo + hi) / 2;
        if (plan_at(mid * kSplitGranule) <= cap) hi = mid;
        else lo = mid + 1;
      }
      plan_at(hi * kSplitGranule);
      const long long cost = k * (rows_per_wg() + kPlanBlockCost);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best_R = hi;
      }
    }
    // no plan within 16 waves: equal rows per workgroup at the fast cap
    plan_at(best_cost < 0 ? kMaxFastChunk : best_R * kSplitGranule);
  }
  const int ns = sa.wt.n > 0 ? sa.wt.cum[sa.wt.n] * sa.Hkv : sa.plan.splits * sa.Hkv * sa.batch_n;
  const int nf = fa.wt.n > 0 ? fa.wt.cum[fa.wt.n] * fa.Hkv : fa.plan.splits * fa.Hkv * fa.batch_n;
  const int sgx = slow_final_blocks(sa, G);
  const int ms = sgx * sa.Hkv * sa.batch_n;
  const int mf = G * fa.Hkv * fa.batch_n;
  const PartialArgs ps = partial_args<D>(sa), pf = partial_args<D>(fa);
  const FinalArgs fs = final_args(sa), ff = final_args(fa);
  hipError_t e;
  if (pend && sa.stats) return hipErrorInvalidValue;  // one selection's key pass per grid
  if (sa.stats && (!sa.evidence || !sa.keysel || sa.nsum)) return hipErrorInvalidValue;
  if (pend) {
    const int np = pend->ws.P * pend->H * pend->batch_n;
    hipLaunchKernelGGL((copartial_kernel<D, G, PAGED, true>), dim3(np + ns + nf), dim3(kThreads), 0, st, ps,
                       pf, sa.plan.splits, fa.plan.splits, sa.Hkv, ns, *pend, np);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((cofinal_kernel<D, G, true>), dim3(np + ms + mf), dim3(kThreads), 0, st, fs, ff, sgx,
                       G, sa.Hkv, ms, *pend, np);
    return hipGetLastError();
  }
  if (ns + nf > 0) {
    if (sa.stats)
      hipLaunchKernelGGL((copartial_kernel<D, G, PAGED, false, true>), dim3(ns + nf), dim3(kThreads), 0, st, ps,
                         pf, sa.plan.splits, fa.plan.splits, sa.Hkv, ns, SelectLaunch{}, 0);
    else
      hipLaunchKernelGGL((copartial_kernel<D, G, PAGED, false>), dim3(ns + nf), dim3(kThreads), 0, st, ps, pf,
                         sa.plan.splits, fa.plan.splits, sa.Hkv, ns, SelectLaunch{}, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (fs.keys)
      hipLaunchKernelGGL((cofinal_kernel<D, G, false, true>), dim3(ms + mf), dim3(kThreads), 0, st, fs, ff, sgx,
                         G, sa.Hkv, ms, SelectLaunch{}, 0);
    else
      hipLaunchKernelGGL((cofinal_kernel<D, G, false>), dim3(ms + mf), dim3(kThreads), 0, st, fs, ff, sgx, G,
                         sa.Hkv, ms, SelectLaunch{}, 0);
  }
  return hipGetLastError();
}

#define SFI_DISPATCH(FN, a, st)                                                   \
  do {                                                                            \
    const bool pg = (a).paged;                                                    \
    switch ((a).d * 16 + (a).G) {                                                 \
      case 64 * 16 + 1: return pg ? FN<64, 1, true>(a, st) : FN<64, 1, false>(a, st);     \
      case 64 * 16 + 2: return pg ? FN<64, 2, true>(a, st) : FN<64, 2, false>(a, st);     \
      case 64 * 16 + 4: return pg ? FN<64, 4, true>(a, st) : FN<64, 4, false>(a, st);     \
      case 64 * 16 + 5: return pg ? FN<64, 5, true>(a, st) : FN<64, 5, false>(a, st);     \
      case 64 * 16 + 8: return pg ? FN<64, 8, true>(a, st) : FN<64, 8, false>(a, st);     \
      case 128 * 16 + 1: return pg ? FN<128, 1, true>(a, st) : FN<128, 1, false>(a, st);  \
      case 128 * 16 + 2: return pg ? FN<128, 2, true>(a, st) : FN<128, 2, false>(a, st);  \
      case 128 * 16 + 4: return pg ? FN<128, 4, true>(a, st) : FN<128, 4, false>(a, st);  \
      case 128 * 16 + 5: return pg ? FN<128, 5, true>(a, st) : FN<128, 5, false>(a, st);  \
      case 128 * 16 + 8: return pg ? FN<128, 8, true>(a, st) : FN<128, 8, false>(a, st);  \
      default: return hipErrorInvalidValue;                                      \
    }                                                                             \
  } while (0)

}  // namespace

int device_cu_count() {
  static int cus[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (cus[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 256;
    cus[dev] = c;
  }
  return cus[dev];
}

SplitPlan plan_splits(long long L, int pairs, int slots, int stride, int max_chunk, bool whole_waves) {
  SplitPlan pl{};
  if (L < 1) L = 1;
  if (pairs < 1) pairs = 1;
  long long want = slots / pairs;  // splits per pair: fill the resident slots at most once
  const long long by_rows = (L + kSplitGranule - 1) / kSplitGranule;
  if (want > by_rows) want = by_rows;
  if (want > stride) want = stride;
  if (want < 1) want = 1;
  long long chunk = (L + want - 1) / want;
  chunk = (chunk + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
  if (chunk > max_chunk && whole_waves) {
    // more splits than one wave of workgroups holds: take whole waves (for
    // dense streams a wave plus a small tail of capped workgroups measured
    // slower than two full waves), then the chunk that spreads L over them
    const long long need = (L + max_chunk - 1) / max_chunk;
    const long long waves = (need + want - 1) / want;
    long long sp = std::min<long long>(waves * want, stride);
    chunk = (L + sp - 1) / sp;
    chunk = (chunk + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
  }
  if (chunk > max_chunk) chunk = max_chunk;
  long long splits = (L + chunk - 1) / chunk;
  if (splits > stride) {  // cannot happen for strides from split_stride(), kept as a guard
    splits = stride;
    chunk = (L + splits - 1) / splits;
  }
  pl.chunk = (int)chunk;
  pl.splits = (int)splits;
  pl.stride = stride;
  return pl;
}

SplitPlan plan_rows(long long L, int stride, long long R, int max_chunk) {
  SplitPlan pl{};
  if (L < 1) L = 1;
  if (stride < 1) stride = 1;
  long long chunk = std::max(R, (L + stride - 1) / stride);
  chunk = (chunk + kSplitGranule - 1) / kSplitGranule * kSplitGranule;
  if (chunk > max_chunk) chunk = max_chunk;
  long long splits = (L + chunk - 1) / chunk;
  if (splits > stride) {  // only when max_chunk binds; kept as a guard
    splits = stride;
    chunk = (L + splits - 1) / splits;
  }
  pl.chunk = (int)chunk;
  pl.splits = (int)splits;
  pl.stride = stride;
  return pl;
}

hipError_t launch_slow(const AttnLaunch &a, hipStream_t st) { SFI_DISPATCH(slow_t, a, st); }
hipError_t launch_step(const AttnLaunch &sa, const AttnLaunch &fa, hipStream_t st, const SelectLaunch *pend) {
  const bool pg = sa.paged;
  switch (sa.d * 16 + sa.G) {
    case 64 * 16 + 1: return pg ? step_t<64, 1, true>(sa, fa, st, pend) : step_t<64, 1, false>(sa, fa, st, pend);
    case 64 * 16 + 2: return pg ? step_t<64, 2, true>(sa, fa, st, pend) : step_t<64, 2, false>(sa, fa, st, pend);
    case 64 * 16 + 4: return pg ? step_t<64, 4, true>(sa, fa, st, pend) : step_t<64, 4, false>(sa, fa, st, pend);
    case 64 * 16 + 5: return pg ? step_t<64, 5, true>(sa, fa, st, pend) : step_t<64, 5, false>(sa, fa, st, pend);
    case 64 * 16 + 8: return pg ? step_t<64, 8, true>(sa, fa, st, pend) : step_t<64, 8, false>(sa, fa, st, pend);
    case 128 * 16 + 1: return pg ? step_t<128, 1, true>(sa, fa, st, pend) : step_t<128, 1, false>(sa, fa, st, pend);
    case 128 * 16 + 2: return pg ? step_t<128, 2, true>(sa, fa, st, pend) : step_t<128, 2, false>(sa, fa, st, pend);
    case 128 * 16 + 4: return pg ? step_t<128, 4, true>(sa, fa, st, pend) : step_t<128, 4, false>(sa, fa, st, pend);
    case 128 * 16 + 5: return pg ? step_t<128, 5, true>(sa, fa, st, pend) : step_t<128, 5, false>(sa, fa, st, pend);
    case 128 * 16 + 8: return pg ? step_t<128, 8, true>(sa, fa, st, pend) : step_t<128, 8, false>(sa, fa, st, pend);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fast(const AttnLaunch &a, hipStream_t st) {
  SFI_DISPATCH(fast_t, a, st);
}

SplitPlan plan_fast(const AttnLaunch &a) {
  switch (a.d * 16 + a.G) {
    case 64 * 16 + 1: return fast_plan_t<64, 1>(a);
    case 64 * 16 + 2: return fast_plan_t<64, 2>(a);
    case 64 * 16 + 4: return fast_plan_t<64, 4>(a);
    case 64 * 16 + 5: return fast_plan_t<64, 5>(a);
    case 64 * 16 + 8: return fast_plan_t<64, 8>(a);
    case 128 * 16 + 1: return fast_plan_t<128, 1>(a);
    case 128 * 16 + 2: return fast_plan_t<128, 2>(a);
    case 128 * 16 + 4: return fast_plan_t<128, 4>(a);
    case 128 * 16 + 5: return fast_plan_t<128, 5>(a);
    case 128 * 16 + 8: return fast_plan_t<128, 8>(a);
    default: return SplitPlan{1, 1, 1};
  }
}

hipError_t launch_fast_compact(const AttnLaunch &a, hipStream_t st) {
  SFI_DISPATCH(fast_compact_t, a, st);
}

hipError_t launch_append(const AttnLaunch &a, const uint16_t *k_new, const uint16_t *v_new, int T,
                         hipStream_t st) {
  if (a.batch_n < 1 || T < 1) return hipSuccess;
  const int slices = T * a.Hkv * (a.d / 8);
  dim3 grid((slices + kThreads - 1) / kThreads, a.batch_n);
#define SFI_APPEND(D_, P_) \
  hipLaunchKernelGGL((append_kernel<D_, P_>), grid, dim3(kThreads), 0, st, a.kv, a.seq_len, a.batch_ids, a.B, \
                     a.max_len, k_new, v_new, T)
  if (a.d == 128) { if (a.paged) SFI_APPEND(128, true); else SFI_APPEND(128, false); }
  else if (a.d == 64) { if (a.paged) SFI_APPEND(64, true); else SFI_APPEND(64, false); }
  else return hipErrorInvalidValue;
#undef SFI_APPEND
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.kv.nstat == nullptr) return e;
  const dim3 g2(a.Hkv, a.batch_n);
  if (a.d == 128)
    hipLaunchKernelGGL(norm_add_kernel<128>, g2, dim3(64), 0, st, a.kv.nstat, a.seq_len, a.batch_ids, a.B, a.Hkv,
                       a.max_len, k_new, T);
  else
    hipLaunchKernelGGL(norm_add_kernel<64>, g2, dim3(64), 0, st, a.kv.nstat, a.seq_len, a.batch_ids, a.B, a.Hkv,
                       a.max_len, k_new, T);
  return hipGetLastError();
}

hipError_t launch_compact(const AttnLaunch &a, uint16_t *ck, uint16_t *cv, hipStream_t st) {
  if (a.sel_k < 1 || a.batch_n < 1) return hipSuccess;
  if (a.d == 128) return a.paged ? compact_t<128, true>(a, ck, cv, st) : compact_t<128, false>(a, ck, cv, st);
  if (a.d == 64) return a.paged ? compact_t<64, true>(a, ck, cv, st) : compact_t<64, false>(a, ck, cv, st);
  return hipErrorInvalidValue;
}

}  // namespace sfi
