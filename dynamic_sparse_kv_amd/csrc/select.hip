// Training-free selector on gfx950, spread over the whole chip.
//
// Slow-Fast Inference (technical summary section 3.B; Korean summary section
// 2.B): the slow step's evidence f is fused with a prior r built from cache
// statistics (key norms and positions) by the reverse-KL objective whose
// minimiser is the mixture s = (1 - lambda) f + lambda r; the Top-K of s over
// the selectable keys becomes the next selected memory.  Vegas (section 2.A)
// ranks aggregated verify logits the same way, with one list per sequence.
//
// A selector row (sequence, head row) is cut into chunks of 2048 keys, one
// 256-thread workgroup per chunk, so every pass over a row's keys runs on
// ~16 compute units per row instead of one.  Each step that needs a row-wide
// result is a kernel boundary (no workgroup ever waits for another):
//   1. norm sums (fused)  per-chunk sum and sum of squares of the key norms
//                         (fp64);
//   2. prior     (fused)  mean and population std from the chunk sums (fixed
//                         order), prior weights w_j and their per-chunk sums;
//                         also clears the row's histogram;
//   3. keys               s_j = (1 - lambda) f_j + lambda w_j / sum(w) as an
//                         order-preserving 32-bit key; the chunk's candidate
//                         keys are bucket-sorted in LDS (4096 buckets, 64 per
//                         octave over the range the scores take) and written (one
//                         coalesced pass) as 64-bit (key, inverted index)
//                         composites in descending bucket order, with the
//                         chunk's cumulative bucket counts; the bucket counts
//                         are merged into the row histogram with integer
//                         atomics;
//   4. pick (per chunk)   every chunk workgroup reads the row histogram and
//                         finds the bucket b1 holding the k-th largest key;
//                         the bucket's keys (a contiguous run in each chunk)
//                         are gathered and radix-selected to the composite
//                         threshold T (the index part makes lower indices win
//                         ties).  Keys in buckets above b1 and bucket keys
//                         >= T win.  Per-chunk winner counts give each chunk
//                         its output offset, and the chunk writes its winners
//                         in ascending index order through an LDS bitmap.
//   The threshold search is repeated by every chunk of the row, which costs
//   O(candidates in b1) per workgroup and saves a launch.
// Integer atomics only build histograms and reserve bucket slots, and every
// floating-point sum runs in a fixed order, so results are bitwise
// repeatable (the order of keys inside a bucket does not affect any result).
#include <algorithm>

#include "select_body.hpp"

namespace sfi {
namespace {

// ---------------------------------------------------------------- 1. sums
__global__ __launch_bounds__(kT) void norm_sums_kernel(SelectLaunch a) {
  __shared__ double s_red[kTW];
  const PairBlock pb = pair_block(linear_block(), gridDim.x, gridDim.y, gridDim.z);
  RowGeo r;
  if (!row_geo(a, pb.h, pb.z, r)) return;
  const int p = pb.blk, j0 = p * kCH;
  if (j0 >= r.n) return;
  const float *nu = a.key_norm + r.row * a.ld;
  float x[kPT];
  load_chunk(nu, j0, r.n, aligned16(nu) && (a.ld & 3) == 0, x);
  double s1 = 0.0, s2 = 0.0;
#pragma unroll
  for (int i = 0; i < kPT; ++i) {
    s1 += (double)x[i];
    s2 += (double)x[i] * (double)x[i];
  }
  s1 = block_sum_d<kTW>(s1, s_red);
  s2 = block_sum_d<kTW>(s2, s_red);
  if (threadIdx.x == 0) {
    a.ws.nsum[(r.row * a.ws.P + p) * 2 + 0] = s1;
    a.ws.nsum[(r.row * a.ws.P + p) * 2 + 1] = s2;
  }
}

// -------------------------------------------------------------- 2. prior
template <bool FUSED>
__global__ __launch_bounds__(kT) void prior_kernel(SelectLaunch a) {
  __shared__ double s_red[kTW];
  const PairBlock pb = pair_block(linear_block(), gridDim.x, gridDim.y, gridDim.z);
  RowGeo r;
  if (!row_geo(a, pb.h, pb.z, r)) return;
  const int p = pb.blk, j0 = p * kCH;
  const int tid = threadIdx.x;
  // clear the row histogram (striped over all chunk workgroups) for step 3
  uint32_t *h1 = a.ws.ghist + r.row * kBins1;
  for (int i = p * kT + tid; i < kBins1; i += a.ws.P * kT) h1[i] = 0u;
  if constexpr (FUSED) {
    if (j0 >= r.n) return;
    const float *nu = a.key_norm + r.row * a.ld;
    float x[kPT];
    load_chunk(nu, j0, r.n, aligned16(nu) && (a.ld & 3) == 0, x);
    const int Pn = (r.n + kCH - 1) / kCH;
    double s1 = 0.0, s2 = 0.0;
    for (int q = tid; q < Pn; q += kT) {
      s1 += a.ws.nsum[(r.row * a.ws.P + q) * 2 + 0];
      s2 += a.ws.nsum[(r.row * a.ws.P + q) * 2 + 1];
    }
    s1 = block_sum_d<kTW>(s1, s_red);
    s2 = block_sum_d<kTW>(s2, s_red);
    float muf, cz;
    prior_consts(s1, s2, r.n, a.norm_coef, &muf, &cz);
    const float ct = kLog2e / a.pos_tau;
    const float tq = (float)(r.n - 1);
    float sw = 0.f;
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
      const int j = key_pos(j0, i);
      sw += (j < r.n) ? prior_w(x[i], j, muf, cz, tq, ct) : 0.f;
    }
    const double W = block_sum_d<kTW>((double)sw, s_red);
    if (tid == 0) {
      a.ws.wsum[r.row * a.ws.P + p] = W;
      if (p == 0) {
        a.ws.meta[r.row].muf = muf;
        a.ws.meta[r.row].cz = cz;
      }
    }
  }
}

// --------------------------------------------------------------- 3. keys
template <bool FUSED, bool REFINE>
__global__ __launch_bounds__(kT) void keys_kernel(SelectLaunch a) {
  const PairBlock pb = pair_block(linear_block(), gridDim.x, gridDim.y, gridDim.z);
  keys_body<FUSED, REFINE>(a, pb.blk, pb.h, pb.z);
}

// ----------------------------------------------------------- 4. pick
__global__ __launch_bounds__(kT) void pick_kernel(SelectLaunch a) {
  const PairBlock pb = pair_block(linear_block(), gridDim.x, gridDim.y, gridDim.z);
  pick_body(a, pb.blk, pb.h, pb.z);
}

}  // namespace

hipError_t launch_select(const SelectLaunch &a, hipStream_t st) {
  const dim3 grid(a.ws.P, a.H, a.batch_n);
  const bool fused = a.mode == 0;
  const bool refine = a.nms_radius > 0 || (a.excl_beta > 0.f && a.H > 1);
  auto keys = [&](const SelectLaunch &x) {
    if (fused && refine)
      hipLaunchKernelGGL((keys_kernel<true, true>), grid, dim3(kT), 0, st, x);
    else if (fused)
      hipLaunchKernelGGL((keys_kernel<true, false>), grid, dim3(kT), 0, st, x);
    else if (refine)
      hipLaunchKernelGGL((keys_kernel<false, true>), grid, dim3(kT), 0, st, x);
    else
      hipLaunchKernelGGL((keys_kernel<false, false>), grid, dim3(kT), 0, st, x);
  };
  hipError_t e;
  if (fused) {
    if (!a.prior_done) {  // else the slow step's finalize wrote the prior sums
      hipLaunchKernelGGL(norm_sums_kernel, grid, dim3(kT), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(prior_kernel<true>, grid, dim3(kT), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    keys(a);
  } else {
    hipLaunchKernelGGL(prior_kernel<false>, grid, dim3(kT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    keys(a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(pick_kernel, grid, dim3(kT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.excl_beta > 0.f && a.H > 1) {
    // exclusivity: the first round's key pass cleared the counts and the
    // second histograms, its pick pass filled the counts and bits; select
    // again with the penalty
    SelectLaunch a2 = a;
    a2.round = 1;
    a2.ws.ghist = a.excl_ghist;
    keys(a2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pick_kernel, grid, dim3(kT), 0, st, a2);
  }
  return hipGetLastError();
}

hipError_t launch_pick(const SelectLaunch &a, hipStream_t st) {
  hipLaunchKernelGGL(pick_kernel, dim3(a.ws.P, a.H, a.batch_n), dim3(kT), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfi
