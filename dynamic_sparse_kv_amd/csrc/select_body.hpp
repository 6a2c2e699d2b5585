// Selector key and pick passes as device functions, so that the selector's
// kernels and the decode kernels that co-launch a pending selection (the
// cross-layer pipeline of sfi_decode_layer_step) run the same code.  See
// select.hip for the design of the chunk-parallel selector.
#pragma once

#include "sfi_internal.hpp"

namespace sfi {
namespace {

constexpr int kT = 256;                 // threads of a chunk workgroup
constexpr int kTW = kT / 64;
constexpr int kCH = kSelChunk;          // keys per chunk
constexpr int kQuarter = kCH / 2;       // keys per half chunk (4 per thread)
constexpr int kPT = kCH / kT;           // keys per thread
constexpr int kD1 = 12;                 // first-level buckets: 4096
constexpr int kBins1 = 1 << kD1;
// Buckets: key bits 30..17 of a positive score (the float's exponent and
// its top 6 mantissa bits) less a base, 64 buckets per octave: from 2^-63
// (bucket 1) to 2^0 (bucket 4033) for fused scores, from 2^-31 to 2^33 for
// raw ones (Vegas' aggregated logits).
constexpr int kFineShift = 17;
constexpr int kFineBase = (64 << 6) - 1;
constexpr int kRawBase = (96 << 6) - 1;
constexpr int kBPT = kBins1 / kT;       // buckets per thread
constexpr int kD2 = 11;                 // digit width inside the bucket
constexpr int kBins2 = 1 << kD2;
// Bucket candidates staged in LDS by the pick (more are read in place from
// the sorted runs; a 32K row's bucket holds ~100).  1024 rather than 4096
// keeps the pick's LDS at 21 KB, so a finalize grid that carries another
// layer's pick keeps 4 waves per SIMD instead of 2 (pipelined 32K headline
// 176.0 -> 178.3-180.7 K tokens/s, 128K stack 2.30 -> 2.36 K).
#ifndef SFI_CAND_LDS
#define SFI_CAND_LDS 1024
#endif
constexpr int kCandLds = SFI_CAND_LDS;  // bucket candidates gathered into LDS (more: read in place)
constexpr int kCPT = kSelMaxChunks / kT;  // chunks per thread in the pick scans
static_assert(kQuarter == 4 * kT, "a half chunk is four keys per thread");
static_assert(kBPT == 16, "sixteen buckets per thread");
static_assert(kCH <= 65535, "cumulative bucket counts are 16-bit");

template <int NW>
__device__ __forceinline__ double block_sum_d(double x, double *s_red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  if (lane == 0) s_red[wv] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += s_red[w];
  __syncthreads();
  return t;
}

// Inclusive prefix sum over the wave in lane order, by DPP: row_shr 1, 2,
// 4, 8 scan each 16-lane row (lanes with no source lane add 0), then
// row_bcast 15 adds the last lane of rows 0 and 2 to rows 1 and 3, and
// row_bcast 31 adds lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Sums of two values over the workgroup (s_pair holds 2 ints per wave).
// Like block_exscan, it ends without a barrier: the next write to s_pair
// must follow another barrier.
template <int NW>
__device__ __forceinline__ void block_sum2(int a, int b, int *s_pair, int *ta, int *tb) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  a = wave_incl_scan(a);
  b = wave_incl_scan(b);
  if (lane == 63) {
    s_pair[2 * wv] = a;
    s_pair[2 * wv + 1] = b;
  }
  __syncthreads();
  int x = 0, y = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    x += s_pair[2 * w];
    y += s_pair[2 * w + 1];
  }
  *ta = x;
  *tb = y;
}

// Exclusive prefix sum over the workgroup in thread order; *total = sum.
// It ends without a barrier: the next write to s_wave must follow another
// barrier (every caller has one before its next scan).
template <int NW>
__device__ __forceinline__ int block_exscan(int v, int *s_wave, int *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = s_wave[w];
    base += (w < wv) ? t : 0;
    tot += t;
  }
  *total = tot;
  return base + x - v;
}

// Row of the selector handled by this workgroup, and its geometry.
// Candidates are [lo, hi); nch chunks hold them (0 when the range is empty).
struct RowGeo {
  int b, h, n, lo, hi, span, nch;
  size_t row;
};

// The geometry of row (b, h) whose clamped length n is known.
__device__ __forceinline__ void row_geo_n(const SelectLaunch &a, int b, int h, int n, RowGeo &r) {
  r.b = b;
  r.h = h;
  r.n = n;
  r.lo = a.n_sink;
  r.hi = max(a.n_sink, r.n - a.window);
  r.span = (a.mode == 0) ? r.n : r.hi;  // keys [0, span) are visited
  r.nch = (r.hi > r.lo) ? (r.hi + kCH - 1) / kCH : 0;
  r.row = (size_t)r.b * a.H + r.h;
}

__device__ __forceinline__ bool row_geo(const SelectLaunch &a, int h, int z, RowGeo &r) {
  r.b = batch_seq(a.batch_ids, z, a.B);
  if (r.b < 0) return false;
  row_geo_n(a, r.b, h, clamp_len(a.seq_len, r.b, a.max_seq_len), r);
  return true;
}

// Key i of thread t in a chunk sits at j0 + (i / 4) * kQuarter + 4 t + i % 4.
__device__ __forceinline__ int key_pos(int j0, int i) {
  return j0 + (i >> 2) * kQuarter + 4 * (int)threadIdx.x + (i & 3);
}

// Values [j0, j0 + kCH) of a row restricted to [0, span) (0 outside).  The
// half-chunk cases are uniform across the workgroup, so no load sits behind a
// per-lane branch: a whole half in range takes one 16-byte load per thread.
// Requires j0 < span.
__device__ __forceinline__ void load_chunk(const float *p, int j0, int span, bool vec,
                                           float (&x)[kPT]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int base = j0 + hf * kQuarter;
    const int j = base + 4 * (int)threadIdx.x;
    if (vec && base + kQuarter <= span) {
      const float4 t = *reinterpret_cast<const float4 *>(p + j);
      x[4 * hf + 0] = t.x; x[4 * hf + 1] = t.y; x[4 * hf + 2] = t.z; x[4 * hf + 3] = t.w;
    } else if (base >= span) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * hf + e] = 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = p[min(j + e, span - 1)];
        x[4 * hf + e] = (j + e < span) ? t : 0.f;
      }
    }
  }
}

__device__ __forceinline__ bool aligned16(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Composite rank value: larger key first, then lower index.
__device__ __forceinline__ unsigned long long composite(uint32_t key, int j) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ __forceinline__ int composite_index(unsigned long long c) {
  return (int)(0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFull));
}

// First-level bucket of a candidate's key: non-decreasing in the key and
// never 0 (the pick reserves bucket 0).  64 buckets per octave over the
// range the scores take (fused: non-negative probability mixtures spread
// over a few dozen octaves; raw: sums of logits, whose top-k sit among the
// positive values), so the k-th largest score's bucket holds about an
// eighth of the keys that a bucket of the key's top 12 bits (sign, exponent
// and 3 mantissa bits) would.  Inside a bucket other than the two end
// buckets the keys share bits 31..17; the end buckets also take what lies
// beyond the range (bucket 1 every negative score).
__device__ __forceinline__ int bucket_base(int mode) { return mode == 0 ? kFineBase : kRawBase; }

__device__ __forceinline__ int key_bucket(uint32_t key, int base) {
  if (!(key & 0x80000000u)) return 1;
  const int v = (int)((key & 0x7FFFFFFFu) >> kFineShift);
  return min(max(v - base, 1), kBins1 - 1);
}

// LDS of the key pass; its histogram is cleared by keys_clear, which a
// caller can issue early (before its own loads are back), with a barrier
// between the clearing and keys_core.
struct KeysLds {
  alignas(16) unsigned hist[kBins1];
  unsigned long long sorted[kCH];
  int wave[kTW];
};

__device__ __forceinline__ void keys_clear(KeysLds &l) {
  for (int i = threadIdx.x; i < kBins1; i += kT) l.hist[i] = 0u;
}

// The key pass of chunk p of a row once its scores are known: s[i] is the
// score of key jj[i] (any assignment of the chunk's keys to threads; the
// candidates are the keys in [r.lo, r.hi)).  Order-preserving 32-bit keys,
// their bucket histogram in LDS merged into the row histogram, the chunk's
// cumulative bucket counts and its bucket-sorted run of (key, inverted
// index) composites.  Every thread of the workgroup calls it.
__device__ __forceinline__ void keys_core(const SelectLaunch &a, const RowGeo &r, int p, const float (&s)[kPT],
                                          const int (&jj)[kPT], KeysLds &l) {
  unsigned *hist = l.hist;
  unsigned long long *s_sorted = l.sorted;
  int *s_wave = l.wave;
  const int tid = threadIdx.x;
  const int base = bucket_base(a.mode);
  uint32_t key[kPT];
  int bk[kPT];
#pragma unroll
  for (int i = 0; i < kPT; ++i) {
    key[i] = (jj[i] >= r.lo && jj[i] < r.hi) ? float_key(s[i]) : 0u;
    bk[i] = key_bucket(key[i], base);
    if (key[i]) atomicAdd(&hist[bk[i]], 1u);
  }
  __syncthreads();
  // Merge the counts into the row histogram first, so the atomics complete
  // while the rest of the pass runs: one 64-bit add per pair of buckets
  // (a count stays far below 2^32, so the low word never carries into the
  // high one), lane t taking pairs t, t + 256, ..., so that one wave's
  // atomics fall on a few adjacent cache lines.
  unsigned long long *h1 = reinterpret_cast<unsigned long long *>(a.ws.ghist + r.row * kBins1);
  const unsigned long long *h64 = reinterpret_cast<const unsigned long long *>(hist);
#pragma unroll
  for (int i = 0; i < kBPT / 2; ++i) {
    const int pr = i * kT + tid;
    const unsigned long long cc = h64[pr];  // buckets 2 pr (low word) and 2 pr + 1
    if (cc) atomicAdd(&h1[pr], cc);
  }
  // Cumulative counts in descending bucket order: cum[b] = keys in buckets
  // >= b.  Thread t owns buckets 16 t .. 16 t + 15.
  uint32_t c[kBPT];
  int tot = 0;
  const uint4 *h4 = reinterpret_cast<const uint4 *>(hist) + (kBPT / 4) * tid;
#pragma unroll
  for (int i = 0; i < kBPT / 4; ++i) {
    const uint4 t = h4[i];
    c[4 * i] = t.x; c[4 * i + 1] = t.y; c[4 * i + 2] = t.z; c[4 * i + 3] = t.w;
  }
#pragma unroll
  for (int i = 0; i < kBPT; ++i) tot += (int)c[i];
  int total;
  const int below = block_exscan<kTW>(tot, s_wave, &total);  // keys in lower buckets
  int run = total - below - tot;                              // keys in higher buckets
  uint32_t cum[kBPT];
#pragma unroll
  for (int i = kBPT - 1; i >= 0; --i) {
    run += (int)c[i];
    cum[i] = (uint32_t)run;
  }
  // bucket b's first slot in the descending layout is cum[b] - count[b]
  uint4 *hw = reinterpret_cast<uint4 *>(hist) + (kBPT / 4) * tid;
#pragma unroll
  for (int i = 0; i < kBPT / 4; ++i)
    hw[i] = make_uint4(cum[4 * i] - c[4 * i], cum[4 * i + 1] - c[4 * i + 1], cum[4 * i + 2] - c[4 * i + 2],
                       cum[4 * i + 3] - c[4 * i + 3]);
  uint4 *cd = reinterpret_cast<uint4 *>(a.ws.cum + (r.row * a.ws.P + p) * kBins1 + kBPT * tid);
  cd[0] = make_uint4(cum[0] | cum[1] << 16, cum[2] | cum[3] << 16, cum[4] | cum[5] << 16,
                     cum[6] | cum[7] << 16);
  cd[1] = make_uint4(cum[8] | cum[9] << 16, cum[10] | cum[11] << 16, cum[12] | cum[13] << 16,
                     cum[14] | cum[15] << 16);
  __syncthreads();
  // bucket sort in LDS, then one coalesced write of the chunk's sorted run
#pragma unroll
  for (int i = 0; i < kPT; ++i) {
    if (key[i]) {
      const unsigned slot = atomicAdd(&hist[bk[i]], 1u);
      s_sorted[slot] = composite(key[i], jj[i]);
    }
  }
  __syncthreads();
  unsigned long long *so = a.ws.sorted + (r.row * a.ws.P + p) * kCH;
  for (int i = tid; i < total; i += kT) so[i] = s_sorted[i];
}


// --------------------------------------------------------------- 3. keys
// Workgroup (chunk p, head row h, batch entry z) of the key pass.
// REFINE = false compiles out Soft-NMS and exclusivity (a call with both
// off runs that variant).
template <bool FUSED, bool REFINE = true>
__device__ __forceinline__ void keys_body(const SelectLaunch &a, int p, int h, int z) {
  __shared__ double s_red[kTW];
  RowGeo r;
  if (!row_geo(a, h, z, r)) return;
  const int j0 = p * kCH;
  const int tid = threadIdx.x;
  const bool excl0 = REFINE && a.excl_beta > 0.f && a.round == 0;
  // exclusivity: the first round clears the second round's row histogram
  if (excl0 && p == 0)
    for (int i = tid; i < kBins1; i += kT) a.excl_ghist[r.row * kBins1 + i] = 0u;
  if (j0 >= r.span) return;

  // Loads issued before the chunk's own work: the Soft-NMS halo keys
  // (kNmsMaxRadius on each side; threads past the halo re-read key j0, so
  // no load sits behind a per-lane branch) and, in exclusivity's second
  // round, the per-key counts and this row's first-round membership bits.
  const bool nms = REFINE && a.nms_radius > 0;
  int hoff = 0;
  float hs = 0.f, hn = 0.f;
  if (nms) {
    hoff = (tid < kNmsMaxRadius) ? tid - kNmsMaxRadius
                                 : (tid < 2 * kNmsMaxRadius ? kCH + tid - kNmsMaxRadius : 0);
    const int jc = min(max(j0 + hoff, 0), r.span - 1);
    hs = a.score[r.row * a.ld + jc];
    if constexpr (FUSED) hn = a.key_norm[r.row * a.ld + jc];
  }
  uint4 ecnt[kPT / 4];
  uint32_t ebit[kPT / 4];
  if (REFINE && a.round == 1) {
    const uint32_t *cnt = a.excl_cnt + (size_t)r.b * a.ld32 * 32;
    const uint32_t *bits = a.excl_bits + r.row * a.ld32;
#pragma unroll
    for (int q = 0; q < kPT / 4; ++q) {
      const int jq = j0 + q * kQuarter + 4 * tid;
      ecnt[q] = *reinterpret_cast<const uint4 *>(cnt + jq);
      ebit[q] = bits[jq >> 5];
    }
  }

  float s[kPT];
  // the fused score's constants (FUSED), kept for the Soft-NMS halo keys
  float cf = 0.f, cr = 0.f, muf = 0.f, cz = 0.f, ct = 0.f, tq = 0.f;
  if constexpr (FUSED) {
    const float *f = a.score + r.row * a.ld;
    const float *nu = a.key_norm + r.row * a.ld;
    const bool vec = aligned16(f) && aligned16(nu) && (a.ld & 3) == 0;
    float fv[kPT], nv[kPT];
    load_chunk(f, j0, r.n, vec, fv);
    load_chunk(nu, j0, r.n, vec, nv);
    const int Pn = (r.n + kCH - 1) / kCH;
    double W = 0.0;
    for (int q = tid; q < Pn; q += kT) W += a.ws.wsum[r.row * a.ws.P + q];
    W = block_sum_d<kTW>(W, s_red);
    cf = 1.0f - a.lambda;
    cr = W > 0.0 ? (float)((double)a.lambda / W) : 0.f;
    muf = a.ws.meta[r.row].muf;
    cz = a.ws.meta[r.row].cz;
    ct = kLog2e / a.pos_tau;
    tq = (float)(r.n - 1);
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
      const int j = key_pos(j0, i);
      const float w = (j < r.n) ? prior_w(nv[i], j, muf, cz, tq, ct) : 0.f;
      s[i] = fmaf(cf, fv[i], cr * w);
    }
    if (a.fused_out) {
      float *fo = a.fused_out + r.row * a.fo_ld;
#pragma unroll
      for (int i = 0; i < kPT; ++i) {
        const int j = key_pos(j0, i);
        if (j < r.n) fo[j] = s[i];
      }
    }
  } else {
    const float *sc = a.score + r.row * a.ld;
    load_chunk(sc, j0, r.span, aligned16(sc) && (a.ld & 3) == 0, s);
  }
  if (p >= r.nch) return;  // no candidates in this chunk
  // exclusivity: the first round clears this chunk's per-key counts (the
  // first-round pick adds to them)
  if (excl0 && h == 0) {
    uint4 *c4 = reinterpret_cast<uint4 *>(a.excl_cnt + (size_t)r.b * a.ld32 * 32 + j0);
#pragma unroll
    for (int q = 0; q < kCH / 4 / kT; ++q) c4[q * kT + tid] = make_uint4(0u, 0u, 0u, 0u);
  }

  // Soft-NMS: a candidate's log score drops by log(1/(1 - alpha)) once per
  // candidate within the radius that ranks above it (larger score, or equal
  // score and lower index).  The chunk's scores and a halo of kNmsMaxRadius
  // keys on each side are staged in LDS; non-candidates never rank above.
  if constexpr (REFINE) {
  if (nms) {
    __shared__ __align__(16) float s_nm[kCH + 2 * kNmsMaxRadius];
    constexpr int HALO = kNmsMaxRadius;
    static_assert(HALO % 4 == 0, "the halo keeps the thread's keys 16-byte aligned");
#pragma unroll
    for (int q = 0; q < kPT / 4; ++q) {
      const int jb = j0 + q * kQuarter + 4 * tid;
      float4 v;
      v.x = (jb >= r.lo && jb < r.hi) ? s[4 * q] : -INFINITY;
      v.y = (jb + 1 >= r.lo && jb + 1 < r.hi) ? s[4 * q + 1] : -INFINITY;
      v.z = (jb + 2 >= r.lo && jb + 2 < r.hi) ? s[4 * q + 2] : -INFINITY;
      v.w = (jb + 3 >= r.lo && jb + 3 < r.hi) ? s[4 * q + 3] : -INFINITY;
      *reinterpret_cast<float4 *>(&s_nm[q * kQuarter + 4 * tid + HALO]) = v;
    }
    if (tid < 2 * HALO) {
      const int j = j0 + hoff;
      float v = -INFINITY;
      if (j >= r.lo && j < r.hi) {
        // the same expression as the chunk's own keys
        if constexpr (FUSED)
          v = fmaf(cf, hs, cr * prior_w(hn, j, muf, cz, tq, ct));
        else
          v = hs;
      }
      s_nm[hoff + HALO] = v;
    }
    __syncthreads();
    const float keep = 1.0f - a.nms_alpha;
    const float lkeep = logf(keep);
    const int R = a.nms_radius;
#pragma unroll
    for (int q = 0; q < kPT / 4; ++q) {
      // s_nm[b0 + t] holds key j0 + q kQuarter + 4 tid - HALO + t
      const int b0 = q * kQuarter + 4 * tid;
      float w[4 + 2 * HALO];
#pragma unroll
      for (int v = 0; v < (4 + 2 * HALO) / 4; ++v) {
        const float4 x = *reinterpret_cast<const float4 *>(&s_nm[b0 + 4 * v]);
        w[4 * v] = x.x;
        w[4 * v + 1] = x.y;
        w[4 * v + 2] = x.z;
        w[4 * v + 3] = x.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + b0 + e;
        const float sj = w[HALO + e];
        int m = 0;
#pragma unroll
        for (int dd = 1; dd <= HALO; ++dd) {
          // lower index: an equal score ranks above
          const int c = (w[HALO + e - dd] >= sj ? 1 : 0) + (w[HALO + e + dd] > sj ? 1 : 0);
          m += (dd <= R) ? c : 0;
        }
        // a penalty of m log(1/keep) on the log score: a factor keep^m on
        // the fused score (a probability), a subtraction on a RAW score
        // (summed logits are already log scores)
        if constexpr (FUSED) {
          float f = 1.0f;
#pragma unroll
          for (int t = 0; t < 2 * HALO; ++t) f = (t < m) ? f * keep : f;
          if (j >= r.lo && j < r.hi) s[4 * q + e] *= f;
        } else {
          if (j >= r.lo && j < r.hi) s[4 * q + e] = fmaf((float)m, lkeep, s[4 * q + e]);
        }
      }
    }
  }
  // Exclusivity's second pass: the log score drops by log(1/(1 - beta))
  // once per other head row of the sequence whose first Top-K holds the key.
  if (a.round == 1) {
    const float keep = 1.0f - a.excl_beta;
    const float lkeep = logf(keep);
#pragma unroll
    for (int q = 0; q < kPT / 4; ++q) {
      const uint32_t c4[4] = {ecnt[q].x, ecnt[q].y, ecnt[q].z, ecnt[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = j0 + q * kQuarter + 4 * tid + e;
        if (j >= r.lo && j < r.hi) {
          const int x = (int)c4[e] - (int)((ebit[q] >> (j & 31)) & 1u);
          if constexpr (FUSED) {
            float f = 1.0f;
            for (int t = 0; t < x; ++t) f *= keep;
            s[4 * q + e] *= f;
          } else {
            s[4 * q + e] = fmaf((float)x, lkeep, s[4 * q + e]);
          }
        }
      }
    }
  }
  }  // REFINE

  int jj[kPT];
#pragma unroll
  for (int i = 0; i < kPT; ++i) jj[i] = key_pos(j0, i);
  __shared__ KeysLds s_keys;
  keys_clear(s_keys);
  __syncthreads();
  keys_core(a, r, p, s, jj, s_keys);
}

// Bin of an nb-bin histogram (nb <= kBins2, highest bin = largest values)
// holding the want-th largest element: s_res = {bin, rank inside it, count}.
// s_res must hold a default before the call; the call ends with a barrier.
__device__ __forceinline__ void find_bin_desc(const unsigned *hist, int nb, int want, int *s_wave,
                                              int *s_res) {
  const int t = threadIdx.x;
  constexpr int BPT = kBins2 / kT;
  const int top = nb - 1 - BPT * t;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) cnt += (top - i >= 0) ? (int)hist[top - i] : 0;
  int total;
  const int above = block_exscan<kTW>(cnt, s_wave, &total);
  if (top >= 0 && above < want && want <= above + cnt) {
    int acc = above;
    for (int i = 0; i < BPT && top - i >= 0; ++i) {
      const int c = (int)hist[top - i];
      if (acc + c >= want) {
        s_res[0] = top - i;
        s_res[1] = want - acc;
        s_res[2] = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

// Cumulative bucket count cum[b] (keys in buckets >= b) of chunk q; 0 for b
// past the last bucket.
__device__ __forceinline__ int cum_at(const SelectLaunch &a, size_t row, int q, int b) {
  return b < kBins1 ? (int)a.ws.cum[(row * a.ws.P + q) * kBins1 + b] : 0;
}

// ----------------------------------------------------------- 4. pick
// Workgroup (chunk p, head row h, batch entry z) of the pick pass.
__device__ __forceinline__ void pick_body(const SelectLaunch &a, int p, int h, int z) {
  __shared__ unsigned h2[kBins2];
  __shared__ unsigned long long s_cand[kCandLds];
  __shared__ int s_above[kSelMaxChunks];   // winners above the bucket, per chunk
  __shared__ int s_toff[kSelMaxChunks + 1];  // bucket candidates before each chunk
  __shared__ int s_tw[kSelMaxChunks];      // bucket winners per chunk
  __shared__ unsigned s_bits[kCH / 32];
  __shared__ int s_wave[kTW];
  __shared__ int s_pair[2 * kTW];
  __shared__ int s_res[3];
  RowGeo r;
  if (!row_geo(a, h, z, r)) return;
  const int tid = threadIdx.x;
  if (p >= max(r.nch, 1)) return;
  const int Kcap = a.k;  // row stride of the index lists
  const int K = a.k_seq ? min(max(a.k_seq[r.b], 0), Kcap) : Kcap;
  int32_t *out = a.sel_idx + r.row * Kcap;
  const unsigned long long *srow = a.ws.sorted + r.row * a.ws.P * kCH;

  // this chunk's bucket-sorted composites (slots past its candidates unused)
  unsigned long long own[kPT];
#pragma unroll
  for (int i = 0; i < kPT; ++i) own[i] = (p < r.nch) ? srow[p * kCH + tid + kT * i] : 0ull;

  // 1. Bucket b1 holding the K-th largest key; thread t holds buckets
  //    16 t .. 16 t + 15 of the row histogram.
  uint32_t hb[kBPT];
  {
    const uint4 *hp = reinterpret_cast<const uint4 *>(a.ws.ghist + r.row * kBins1 + kBPT * tid);
#pragma unroll
    for (int i = 0; i < kBPT / 4; ++i) {
      const uint4 v = hp[i];
      hb[4 * i] = v.x; hb[4 * i + 1] = v.y; hb[4 * i + 2] = v.z; hb[4 * i + 3] = v.w;
    }
  }
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < kBPT; ++i) cnt += (int)hb[i];
  int total;
  if (tid == 0) {  // default, ordered before the finder's write by the scan's barrier
    s_res[0] = 0;  // b1 = 0: every candidate wins (candidate keys never sit in bucket 0)
    s_res[1] = 0;
    s_res[2] = 0;
  }
  const int below = block_exscan<kTW>(cnt, s_wave, &total);
  const int above = total - below - cnt;
  if (total > K && above < K && K <= above + cnt) {
    int acc = above;
    for (int i = kBPT - 1; i >= 0; --i) {
      const int c = (int)hb[i];
      if (acc + c >= K) {
        s_res[0] = kBPT * tid + i;
        s_res[1] = K - acc;
        s_res[2] = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  const int b1 = s_res[0];
  const int want1 = s_res[1];
  const int m = s_res[2];
  const bool split = b1 != 0 && want1 < m;  // only part of bucket b1 wins

  // 2. Per chunk: winners above the bucket (a prefix of its sorted run) and
  //    its run of bucket-b1 keys.  Thread t handles chunks kCPT t ...
  int na[kCPT], nt[kCPT];
  int tsum = 0;
#pragma unroll
  for (int i = 0; i < kCPT; ++i) {
    const int q = kCPT * tid + i;
    na[i] = nt[i] = 0;
    if (q < r.nch) {
      if (b1 == 0) {
        na[i] = cum_at(a, r.row, q, 0);
      } else if (split) {
        na[i] = cum_at(a, r.row, q, b1 + 1);
        nt[i] = cum_at(a, r.row, q, b1) - na[i];
      } else {
        na[i] = cum_at(a, r.row, q, b1);
      }
      s_above[q] = na[i];
    }
    tsum += nt[i];
  }
  int mtot;
  int toff = block_exscan<kTW>(tsum, s_wave, &mtot);
#pragma unroll
  for (int i = 0; i < kCPT; ++i) {
    const int q = kCPT * tid + i;
    if (q < r.nch) {
      s_toff[q] = toff;
      s_tw[q] = 0;
    }
    toff += nt[i];
  }
  if (tid == 0) s_toff[r.nch] = mtot;
  __syncthreads();

  // 3. Selection of the want1-th largest composite among the m bucket-b1
  //    keys: their ranks when they fit one per thread, else a radix select
  //    with 11-bit digits below the bits the bucket's keys share (bits
  //    63..49; none for an end bucket).  Bucket keys win iff their
  //    composite >= T.
  unsigned long long T = 0ull;
  if (split) {
    const bool in_lds = mtot <= kCandLds;
    // i-th bucket key of the row, in chunk order
    auto cand_at = [&](int i) -> unsigned long long {
      int lo = 0, hi = r.nch - 1;
      while (lo < hi) {  // last chunk q with s_toff[q] <= i
        const int mid = (lo + hi + 1) >> 1;
        if (s_toff[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      return srow[lo * kCH + s_above[lo] + (i - s_toff[lo])];
    };
    if (in_lds) {
      // four candidates per thread per round, their loads in flight together
      for (int i0 = 0; i0 < mtot; i0 += 4 * kT) {
        unsigned long long v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + tid + u * kT;
          v[u] = (i < mtot) ? cand_at(i) : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + tid + u * kT;
          if (i < mtot) s_cand[i] = v[u];
        }
      }
      __syncthreads();
    }
    auto cand = [&](int i) { return in_lds ? s_cand[i] : cand_at(i); };
    if (mtot <= kT) {
      // A candidate's rank among the candidates (the composites are
      // distinct) decides it, and the one of rank want1 - 1 is the
      // threshold.  Up to 64 candidates, 4 adjacent lanes rank one, each
      // over a quarter of the list (2 lanes up to 128); the comparisons go
      // four at a time so the LDS reads overlap.
      __shared__ unsigned long long s_thr;
      const int lg = mtot <= 64 ? 2 : (mtot <= 128 ? 1 : 0);
      const int i = tid >> lg, part = tid & ((1 << lg) - 1);
      const int len = (mtot + (1 << lg) - 1) >> lg;
      const int j0 = part * len, j1 = min(mtot, j0 + len);
      const unsigned long long c = (i < mtot) ? s_cand[i] : 0ull;
      int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
      int j = j0;
      for (; j + 4 <= j1; j += 4) {
        r0 += (s_cand[j] > c) ? 1 : 0;
        r1 += (s_cand[j + 1] > c) ? 1 : 0;
        r2 += (s_cand[j + 2] > c) ? 1 : 0;
        r3 += (s_cand[j + 3] > c) ? 1 : 0;
      }
      for (; j < j1; ++j) r0 += (s_cand[j] > c) ? 1 : 0;
      int rank = (r0 + r1) + (r2 + r3);
      if (lg >= 1) rank += __shfl_xor(rank, 1);
      if (lg >= 2) rank += __shfl_xor(rank, 2);
      if (i < mtot && part == 0 && rank < want1) atomicAdd(&s_tw[min(composite_index(c) / kCH, r.nch - 1)], 1);
      if (i < mtot && part == 0 && rank == want1 - 1) s_thr = c;
      __syncthreads();
      T = s_thr;
    } else {
    unsigned long long prefix = 0ull;
    int top = 63, want = want1;
    if (b1 > 1 && b1 < kBins1 - 1) {
      prefix = 0x4000ull | (unsigned long long)(b1 + bucket_base(a.mode));  // key bits 31..17
      top = 31 + kFineShift;
    }
    for (;;) {
      const int lo_bit = max(top - kD2 + 1, 0);
      const int width = top - lo_bit + 1;
      const unsigned long long dmask = (1ull << width) - 1ull;
      for (int i = tid; i < (1 << width); i += kT) h2[i] = 0u;
      if (tid == 0) {
        s_res[0] = 0;
        s_res[1] = 1;
        s_res[2] = 0;
      }
      __syncthreads();
      for (int i = tid; i < mtot; i += kT) {
        const unsigned long long c = cand(i);
        if (top == 63 || (c >> (top + 1)) == prefix) atomicAdd(&h2[(c >> lo_bit) & dmask], 1u);
      }
      __syncthreads();
      find_bin_desc(h2, 1 << width, want, s_wave, s_res);
      const int bin = s_res[0];
      want = s_res[1];
      const int c = s_res[2];
      __syncthreads();
      prefix = (prefix << width) | (unsigned long long)bin;
      if (lo_bit == 0 || want == c) {  // the whole sub-bin is taken
        T = prefix << lo_bit;
        break;
      }
      top = lo_bit - 1;
    }
    // bucket winners per chunk (the chunk is the key index / chunk size)
    for (int i = tid; i < mtot; i += kT) {
      const unsigned long long c = cand(i);
      if (c >= T) atomicAdd(&s_tw[min(composite_index(c) / kCH, r.nch - 1)], 1);
    }
    __syncthreads();
    }  // radix select
  }

  // 4. Output offset of this chunk (winners of the chunks before it) and
  //    the row's winner count.
  int wb = 0, wt = 0;
#pragma unroll
  for (int i = 0; i < kCPT; ++i) {
    const int q = kCPT * tid + i;
    if (q < r.nch) {
      const int w = s_above[q] + s_tw[q];
      wt += w;
      wb += (q < p) ? w : 0;
    }
  }
  // (the bitmap of step 5 is cleared here, ordered by the sum's barrier)
  if (tid < kCH / 32) s_bits[tid] = 0u;
  int before, total_w;
  block_sum2<kTW>(wb, wt, s_pair, &before, &total_w);
  const int count = min(total_w, K);

  // 5. This chunk's winners, ascending, through a 2048-bit bitmap.
  if (p < r.nch) {
    const int na_p = s_above[p];
    const int ne_p = split ? s_toff[p + 1] - s_toff[p] : 0;
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
      const int slot = tid + kT * i;
      const bool w = slot < na_p || (slot < na_p + ne_p && own[i] >= T);
      if (w) {
        const int jl = composite_index(own[i]) - p * kCH;
        if (jl >= 0 && jl < kCH) atomicOr(&s_bits[jl >> 5], 1u << (jl & 31));
      }
    }
    __syncthreads();
    // thread t owns bits 8 t .. 8 t + 7
    const uint32_t byte = (s_bits[tid >> 2] >> (8 * (tid & 3))) & 0xFFu;
    int tot8;
    int o = before + block_exscan<kTW>(__popc(byte), s_wave, &tot8);
    const bool scat = a.excl_beta > 0.f && a.round == 0;
    uint32_t unw = 0u;  // winners past the list's capacity
    for (int e = 0; e < 8; ++e) {
      if (byte & (1u << e)) {
        const int j = p * kCH + 8 * tid + e;
        if (o < K) {
          out[o] = j;
          if (scat) atomicAdd(&a.excl_cnt[(size_t)r.b * a.ld32 * 32 + j], 1u);
        } else {
          unw |= 1u << e;
        }
        ++o;
      }
    }
    if (scat) {
      // this chunk's words of the row's membership bits (every thread read
      // its byte before the scan's barrier)
      if (unw) atomicAnd(&s_bits[tid >> 2], ~(unw << (8 * (tid & 3))));
      __syncthreads();
      if (tid < kCH / 32) a.excl_bits[r.row * a.ld32 + p * (kCH / 32) + tid] = s_bits[tid];
    }
  }
  // 6. The last chunk's workgroup pads the list and writes its length.
  if (p == max(r.nch, 1) - 1) {
    if (tid == 0) a.sel_count[r.row] = count;
    for (int i = count + tid; i < Kcap; i += kT) out[i] = -1;
  }
}

}  // namespace
}  // namespace sfi
