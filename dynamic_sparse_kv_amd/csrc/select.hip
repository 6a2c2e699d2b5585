// Training-free selector on gfx950.
//
// Slow-Fast Inference (technical summary section 3.B; Korean summary section
// 2.B): the slow step's evidence f is fused with a prior r built from cache
// statistics (key norms and positions) by the reverse-KL objective whose
// minimiser is the mixture s = (1 - lambda) f + lambda r; the Top-K of s over
// the selectable keys becomes the next selected memory.  Vegas (section 2.A)
// ranks aggregated verify logits the same way, with one list per sequence.
//
// Kernels, per (sequence, head row):
//   stats_kernel  - chunked fp64 sums of key norms and squared norms;
//   prior_kernel  - mean/std from those sums (fixed-order merge), unnormalised
//                   prior weights w_j and chunked fp64 sums of w;
//   topk_kernel   - one 1024-thread workgroup: s_j = (1-lambda) f_j +
//                   lambda w_j / sum(w) fused into the first radix pass, a
//                   12/12/8-bit radix select of the k-th largest key in LDS
//                   histograms, then an ordered compaction (ballot-free block
//                   scans) that emits the winners in ascending index order
//                   with ties at the threshold going to the lowest indices.
#include "sfi_internal.hpp"

namespace sfi {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kPerThread = 8;

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ __launch_bounds__(256) void stats_kernel(SelectLaunch a) {
  __shared__ double red[4][2];
  const int b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (b < 0) return;
  const int h = blockIdx.y;
  const int n = clamp_len(a.seq_len, b, a.max_seq_len);
  const int j0 = blockIdx.x * kStatChunk;
  if (j0 >= n) return;
  const int j1 = min(n, j0 + kStatChunk);
  const size_t row = (size_t)b * a.H + h;
  const float *nu = a.key_norm + row * a.ld;
  double s1 = 0.0, s2 = 0.0;
  for (int j = j0 + threadIdx.x; j < j1; j += 256) {
    const double v = nu[j];
    s1 += v;
    s2 += v * v;
  }
  s1 = wave_sum_d(s1);
  s2 = wave_sum_d(s2);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) {
    red[wv][0] = s1;
    red[wv][1] = s2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t1 = 0.0, t2 = 0.0;
    for (int w = 0; w < 4; ++w) {
      t1 += red[w][0];
      t2 += red[w][1];
    }
    a.stats[(row * a.nch + blockIdx.x) * 2 + 0] = t1;
    a.stats[(row * a.nch + blockIdx.x) * 2 + 1] = t2;
  }
}

__global__ __launch_bounds__(256) void prior_kernel(SelectLaunch a) {
  __shared__ double red[4];
  const int b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (b < 0) return;
  const int h = blockIdx.y;
  const int n = clamp_len(a.seq_len, b, a.max_seq_len);
  const int j0 = blockIdx.x * kStatChunk;
  if (j0 >= n) return;
  const int j1 = min(n, j0 + kStatChunk);
  const size_t row = (size_t)b * a.H + h;
  const int nc = (n + kStatChunk - 1) / kStatChunk;
  double t1 = 0.0, t2 = 0.0;
  for (int c = 0; c < nc; ++c) {
    t1 += a.stats[(row * a.nch + c) * 2 + 0];
    t2 += a.stats[(row * a.nch + c) * 2 + 1];
  }
  const double mu = t1 / n;
  const double var = fmax(t2 / n - mu * mu, 0.0);
  const double sd = sqrt(var);
  const float muf = (float)mu;
  const float inv_sd = sd > 0.0 ? (float)(1.0 / sd) : 0.0f;
  const float t = (float)(n - 1);
  const float inv_tau = 1.0f / a.pos_tau;
  const float *nu = a.key_norm + row * a.ld;
  float *w = a.sbuf + row * a.sld;
  double sw = 0.0;
  for (int j = j0 + threadIdx.x; j < j1; j += 256) {
    const float z = (nu[j] - muf) * inv_sd;
    const float wj = expf(-a.norm_coef * z) * (1.0f + expf(-(t - (float)j) * inv_tau));
    w[j] = wj;
    sw += (double)wj;
  }
  sw = wave_sum_d(sw);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (lane == 0) red[wv] = sw;
  __syncthreads();
  if (threadIdx.x == 0) a.wsum[row * a.nch + blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

// Exclusive prefix sum over the 1024 threads in thread order; *total gets the sum.
__device__ __forceinline__ int block_exscan(int v, int *s_wave, int *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wv] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = s_wave[w];
    base += (w < wv) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Given a histogram of NB bins, find the bin holding the want-th largest
// element (want >= 1).  Returns the bin in *bin and the rank left inside it.
template <int NB>
__device__ __forceinline__ void find_bin(const unsigned *hist, int want, int *s_wave,
                                         int *s_res) {
  const int t = threadIdx.x;
  if (t == 0) {
    s_res[0] = 0;
    s_res[1] = 1;
  }
  const int hi = NB - 1 - 4 * t;
  int cnt = 0;
  if (hi >= 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt += (hi - i >= 0) ? (int)hist[hi - i] : 0;
  }
  int total;
  const int above = block_exscan(cnt, s_wave, &total);
  if (hi >= 0 && above < want && want <= above + cnt) {
    int acc = above;
    for (int i = 0; i < 4; ++i) {
      const int c = (int)hist[hi - i];
      if (acc + c >= want) {
        s_res[0] = hi - i;
        s_res[1] = want - acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

template <bool FUSED>
__global__ __launch_bounds__(kSelThreads) void topk_kernel(SelectLaunch a) {
  __shared__ unsigned hist[4096];
  __shared__ int s_wave[kSelWaves];
  __shared__ int s_res[2];

  const int b = batch_seq(a.batch_ids, blockIdx.y, a.B);
  if (b < 0) return;
  const int h = blockIdx.x;
  const int n = clamp_len(a.seq_len, b, a.max_seq_len);
  const int tid = threadIdx.x;
  const size_t row = (size_t)b * a.H + h;
  const int lo = a.n_sink;
  const int hi = max(a.n_sink, n - a.window);
  const int ncand = max(0, hi - lo);
  const int K = a.k;
  int32_t *out = a.sel_idx + row * K;

  // Scores of this row: FUSED writes s into sbuf during the first pass.
  const float *src = FUSED ? (const float *)(a.sbuf + row * a.sld) : a.score + row * a.ld;

  for (int i = tid; i < 4096; i += kSelThreads) hist[i] = 0u;
  __syncthreads();

  if constexpr (FUSED) {
    const int nc = (n + kStatChunk - 1) / kStatChunk;
    double W = 0.0;
    for (int c = 0; c < nc; ++c) W += a.wsum[row * a.nch + c];
    const float cf = 1.0f - a.lambda;
    const float cr = (float)((double)a.lambda / W);
    const float *f = a.score + row * a.ld;
    float *s = a.sbuf + row * a.sld;
    for (int j = tid; j < n; j += kSelThreads) {
      const float v = fmaf(cf, f[j], cr * s[j]);
      s[j] = v;
      if (j >= lo && j < hi && ncand > K) atomicAdd(&hist[float_key(v) >> 20], 1u);
    }
  } else {
    if (ncand > K) {
      for (int j = lo + tid; j < hi; j += kSelThreads) atomicAdd(&hist[float_key(src[j]) >> 20], 1u);
    }
  }
  __syncthreads();

  uint32_t thr = 0u;   // full 32-bit threshold key
  int take_eq = 0;     // how many keys equal to thr are taken (lowest index first)
  const bool take_all = ncand <= K;
  if (!take_all) {
    // pass 1: bits 31..20
    find_bin<4096>(hist, K, s_wave, s_res);
    const uint32_t b1 = (uint32_t)s_res[0];
    int want = s_res[1];
    __syncthreads();
    for (int i = tid; i < 4096; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    // pass 2: bits 19..8 among keys whose top 12 bits equal b1
    for (int j = lo + tid; j < hi; j += kSelThreads) {
      const uint32_t key = float_key(src[j]);
      if ((key >> 20) == b1) atomicAdd(&hist[(key >> 8) & 0xFFFu], 1u);
    }
    __syncthreads();
    find_bin<4096>(hist, want, s_wave, s_res);
    const uint32_t b2 = (uint32_t)s_res[0];
    want = s_res[1];
    __syncthreads();
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0u;
    __syncthreads();
    const uint32_t pre = (b1 << 12) | b2;
    // pass 3: bits 7..0
    for (int j = lo + tid; j < hi; j += kSelThreads) {
      const uint32_t key = float_key(src[j]);
      if ((key >> 8) == pre) atomicAdd(&hist[key & 0xFFu], 1u);
    }
    __syncthreads();
    find_bin<256>(hist, want, s_wave, s_res);
    thr = (pre << 8) | (uint32_t)s_res[0];
    take_eq = s_res[1];
    __syncthreads();
  }

  // Ordered compaction: thread t owns kPerThread consecutive candidates of
  // each tile, so winners come out in ascending index order.
  int carry_eq = 0, carry_sel = 0;
  constexpr int TILE = kSelThreads * kPerThread;
  for (int base = lo; base < hi; base += TILE) {
    const int j0 = base + tid * kPerThread;
    uint32_t keys[kPerThread];
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int j = j0 + i;
      keys[i] = (j < hi) ? float_key(src[j]) : 0u;
      if (j < hi) {
        if (take_all || keys[i] > thr) ++gt;
        else if (keys[i] == thr) ++eq;
      }
    }
    int eq_tot;
    const int eq_base = carry_eq + block_exscan(eq, s_wave, &eq_tot);
    const int take_here = min(max(take_eq - eq_base, 0), eq);
    int sel_tot;
    const int sel_base = carry_sel + block_exscan(gt + take_here, s_wave, &sel_tot);
    int pos = sel_base, er = eq_base;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int j = j0 + i;
      if (j < hi) {
        if (take_all || keys[i] > thr) {
          if (pos < K) out[pos] = j;
          ++pos;
        } else if (keys[i] == thr) {
          if (er < take_eq) {
            if (pos < K) out[pos] = j;
            ++pos;
          }
          ++er;
        }
      }
    }
    carry_eq += eq_tot;
    carry_sel += sel_tot;
  }
  for (int i = carry_sel + tid; i < K; i += kSelThreads) out[i] = -1;
  if (tid == 0) a.sel_count[row] = min(carry_sel, K);
}

}  // namespace

hipError_t launch_select(const SelectLaunch &a, hipStream_t st) {
  if (a.mode == 0) {
    dim3 g1(a.nch, a.H, a.batch_n);
    hipLaunchKernelGGL(stats_kernel, g1, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prior_kernel, g1, dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel<true>, dim3(a.H, a.batch_n), dim3(kSelThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL(topk_kernel<false>, dim3(a.H, a.batch_n), dim3(kSelThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sfi
