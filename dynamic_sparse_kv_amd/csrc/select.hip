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
// 256-thread workgroup per chunk, so a row's loads and arithmetic run on ~16
// compute units instead of one.  Each step that needs a row-wide result is a
// kernel boundary (no workgroup ever waits for another):
//   1. norm sums     (fused)  per-chunk sum and sum of squares of the key
//                             norms (fp64);
//   2. prior         (fused)  mean and population std from the chunk sums
//                             (fixed order), prior weights w_j and their
//                             per-chunk sums; also clears the row's histogram;
//   3. keys                   s_j = (1 - lambda) f_j + lambda w_j / sum(w)
//                             as an order-preserving 32-bit key (0 for keys
//                             outside the candidate range), stored; a
//                             histogram of the top 12 key bits, merged into
//                             the row's histogram with integer atomics;
//   4. tie bin                every chunk finds the bin holding the k-th
//                             largest key from the row histogram; counts its
//                             keys above that bin and appends the keys inside
//                             it, as 64-bit (key, inverted index) composites,
//                             to the row's candidate list;
//   5. threshold (one workgroup per row) radix-selects the composite
//                             threshold T among the candidates (the index part
//                             makes lower indices win ties), then turns
//                             per-chunk winner counts into output offsets;
//   6. compaction             each chunk writes its winners, ascending, at
//                             its offset.
// Integer atomics only build histograms and reserve list slots, and every
// floating-point sum runs in a fixed order, so results are bitwise
// repeatable.
#include "sfi_internal.hpp"

namespace sfi {
namespace {

constexpr int kT = 256;                 // threads of a chunk workgroup
constexpr int kTW = kT / 64;
constexpr int kCH = kSelChunk;          // keys per chunk
constexpr int kHalf = kCH / 2;          // keys per half chunk (4 per thread)
constexpr int kPT = kCH / kT;           // keys per thread
constexpr int kD1 = 12;                 // first digit: key bits 31..20
constexpr int kBins1 = 1 << kD1;
constexpr int kRT = 1024;               // threads of the threshold workgroup
constexpr int kRW = kRT / 64;
constexpr int kD2 = 11;                 // digit width inside the tie bin
constexpr int kBins2 = 1 << kD2;
static_assert(kHalf == 4 * kT, "a half chunk is four keys per thread");

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

// Exclusive prefix sum over the workgroup in thread order; *total = sum.
template <int NW>
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
  for (int w = 0; w < NW; ++w) {
    const int t = s_wave[w];
    base += (w < wv) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Row of the selector handled by this workgroup, and its geometry.
struct RowGeo {
  int b, h, n, lo, hi, span;
  size_t row;
};

__device__ __forceinline__ bool row_geo(const SelectLaunch &a, RowGeo &r) {
  r.b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (r.b < 0) return false;
  r.h = blockIdx.y;
  r.n = clamp_len(a.seq_len, r.b, a.max_seq_len);
  r.lo = a.n_sink;
  r.hi = max(a.n_sink, r.n - a.window);
  r.span = (a.mode == 0) ? r.n : r.hi;  // keys [0, span) are visited
  r.row = (size_t)r.b * a.H + r.h;
  return true;
}

// Key i of thread t in a chunk sits at j0 + (i / 4) * kHalf + 4 t + i % 4.
__device__ __forceinline__ int key_pos(int j0, int i) {
  return j0 + (i >> 2) * kHalf + 4 * (int)threadIdx.x + (i & 3);
}

// Values [j0, j0 + kCH) of a row restricted to [0, span) (0 outside).  The
// half-chunk cases are uniform across the workgroup, so no load sits behind a
// per-lane branch: a whole half in range takes one 16-byte load per thread.
__device__ __forceinline__ void load_chunk(const float *p, int j0, int span, bool vec,
                                           float (&x)[kPT]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int base = j0 + hf * kHalf;
    const int j = base + 4 * (int)threadIdx.x;
    if (vec && base + kHalf <= span) {
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

__device__ __forceinline__ void load_keys(const uint32_t *p, int j0, uint32_t (&k)[kPT]) {
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const uint4 t = *reinterpret_cast<const uint4 *>(p + j0 + hf * kHalf + 4 * threadIdx.x);
    k[4 * hf + 0] = t.x; k[4 * hf + 1] = t.y; k[4 * hf + 2] = t.z; k[4 * hf + 3] = t.w;
  }
}

__device__ __forceinline__ bool aligned16(const void *p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Prior weight of key j: exp(-norm_coef z_j) (1 + exp(-(t - j)/tau)) with
// z_j = (nu_j - mu)/sd, as powers of two (cz = -norm_coef log2(e)/sd,
// ct = log2(e)/tau).  Steps 2 and 3 both call it, so the weights and their sum
// agree bit for bit.
__device__ __forceinline__ float prior_w(float nu, int j, float muf, float cz, float tq, float ct) {
  return exp2f(cz * (nu - muf)) * (1.0f + exp2f(((float)j - tq) * ct));
}

// Composite rank value: larger key first, then lower index.
__device__ __forceinline__ unsigned long long composite(uint32_t key, int j) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)j);
}

// ---------------------------------------------------------------- 1. sums
__global__ __launch_bounds__(kT) void norm_sums_kernel(SelectLaunch a) {
  __shared__ double s_red[kTW];
  RowGeo r;
  if (!row_geo(a, r)) return;
  const int p = blockIdx.x, j0 = p * kCH;
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
  RowGeo r;
  if (!row_geo(a, r)) return;
  const int p = blockIdx.x, j0 = p * kCH;
  const int tid = threadIdx.x;
  // clear the row's histogram (striped over all chunk workgroups) and its
  // candidate counter, for steps 3 and 4
  uint32_t *h1 = a.ws.hist + r.row * kBins1;
  for (int i = p * kT + tid; i < kBins1; i += a.ws.P * kT) h1[i] = 0u;
  if (p == 0 && tid == 0) a.ws.meta[r.row].m = 0;
  if constexpr (FUSED) {
    if (j0 >= r.n) return;
    const int Pn = (r.n + kCH - 1) / kCH;
    double s1 = 0.0, s2 = 0.0;
    for (int q = tid; q < Pn; q += kT) {
      s1 += a.ws.nsum[(r.row * a.ws.P + q) * 2 + 0];
      s2 += a.ws.nsum[(r.row * a.ws.P + q) * 2 + 1];
    }
    s1 = block_sum_d<kTW>(s1, s_red);
    s2 = block_sum_d<kTW>(s2, s_red);
    const double mu = s1 / r.n;
    const double var = fmax(s2 / r.n - mu * mu, 0.0);
    const double sd = sqrt(var);
    const float muf = (float)mu;
    const float isd = sd > 0.0 ? (float)(1.0 / sd) : 0.0f;
    const float cz = -a.norm_coef * isd * kLog2e;
    const float ct = kLog2e / a.pos_tau;
    const float tq = (float)(r.n - 1);
    const float *nu = a.key_norm + r.row * a.ld;
    float x[kPT];
    load_chunk(nu, j0, r.n, aligned16(nu) && (a.ld & 3) == 0, x);
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
template <bool FUSED>
__global__ __launch_bounds__(kT) void keys_kernel(SelectLaunch a) {
  __shared__ unsigned hist[kBins1];
  __shared__ double s_red[kTW];
  RowGeo r;
  if (!row_geo(a, r)) return;
  const int p = blockIdx.x, j0 = p * kCH;
  if (j0 >= r.span) return;
  const int tid = threadIdx.x;
  for (int i = tid; i < kBins1; i += kT) hist[i] = 0u;

  float s[kPT];
  if constexpr (FUSED) {
    const int Pn = (r.n + kCH - 1) / kCH;
    double W = 0.0;
    for (int q = tid; q < Pn; q += kT) W += a.ws.wsum[r.row * a.ws.P + q];
    W = block_sum_d<kTW>(W, s_red);
    const float cf = 1.0f - a.lambda;
    const float cr = W > 0.0 ? (float)((double)a.lambda / W) : 0.f;
    const float muf = a.ws.meta[r.row].muf, cz = a.ws.meta[r.row].cz;
    const float ct = kLog2e / a.pos_tau;
    const float tq = (float)(r.n - 1);
    const float *f = a.score + r.row * a.ld;
    const float *nu = a.key_norm + r.row * a.ld;
    const bool vec = aligned16(f) && aligned16(nu) && (a.ld & 3) == 0;
    float fv[kPT], nv[kPT];
    load_chunk(f, j0, r.n, vec, fv);
    load_chunk(nu, j0, r.n, vec, nv);
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
  uint32_t key[kPT];
#pragma unroll
  for (int i = 0; i < kPT; ++i) {
    const int j = key_pos(j0, i);
    key[i] = (j >= r.lo && j < r.hi) ? float_key(s[i]) : 0u;
  }
  uint32_t *kp = a.ws.keys + r.row * a.ws.ldk + j0;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    *reinterpret_cast<uint4 *>(kp + hf * kHalf + 4 * tid) =
        make_uint4(key[4 * hf], key[4 * hf + 1], key[4 * hf + 2], key[4 * hf + 3]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPT; ++i)
    if (key[i]) atomicAdd(&hist[key[i] >> (32 - kD1)], 1u);
  __syncthreads();
  uint32_t *h1 = a.ws.hist + r.row * kBins1;
  for (int i = tid; i < kBins1; i += kT) {
    const unsigned c = hist[i];
    if (c) atomicAdd(&h1[i], c);
  }
}

// ----------------------------------------------------------- 4. tie bin
__global__ __launch_bounds__(kT) void tie_kernel(SelectLaunch a) {
  __shared__ int s_wave[kTW];
  __shared__ int s_res[3];
  __shared__ int s_base;
  RowGeo r;
  if (!row_geo(a, r)) return;
  const int p = blockIdx.x, j0 = p * kCH;
  if (j0 >= r.span) return;
  const int tid = threadIdx.x;
  const int K = a.k;

  // The row histogram: thread t holds bins BPT t .. BPT t + BPT - 1.
  constexpr int BPT = kBins1 / kT;
  const uint32_t *h1 = a.ws.hist + r.row * kBins1 + BPT * tid;
  uint32_t hb[BPT];
#pragma unroll
  for (int i = 0; i < BPT; i += 4) {
    const uint4 t = *reinterpret_cast<const uint4 *>(h1 + i);
    hb[i] = t.x; hb[i + 1] = t.y; hb[i + 2] = t.z; hb[i + 3] = t.w;
  }
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) cnt += (int)hb[i];
  int total;
  const int below = block_exscan<kTW>(cnt, s_wave, &total);  // keys in lower bins
  if (tid == 0) {
    s_res[0] = 0;  // b1 = 0 takes every candidate (their top digit is > 0)
    s_res[1] = 0;
    s_res[2] = 0;
  }
  __syncthreads();
  const int above = total - below - cnt;
  if (total > K && above < K && K <= above + cnt) {
    int acc = above;
    for (int i = BPT - 1; i >= 0; --i) {
      const int c = (int)hb[i];
      if (acc + c >= K) {
        s_res[0] = BPT * tid + i;
        s_res[1] = K - acc;
        s_res[2] = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  const uint32_t b1 = (uint32_t)s_res[0];
  if (p == 0 && tid == 0) {
    a.ws.meta[r.row].b1 = (int)b1;
    a.ws.meta[r.row].want1 = s_res[1];
  }

  uint32_t key[kPT];
  load_keys(a.ws.keys + r.row * a.ws.ldk, j0, key);
  int gt = 0, ne = 0;
#pragma unroll
  for (int i = 0; i < kPT; ++i) {
    const uint32_t d = key[i] >> (32 - kD1);
    gt += (key[i] != 0u && d > b1) ? 1 : 0;
    ne += (key[i] != 0u && b1 != 0u && d == b1) ? 1 : 0;
  }
  int gtot;
  block_exscan<kTW>(gt, s_wave, &gtot);
  int etot;
  const int eoff = block_exscan<kTW>(ne, s_wave, &etot);
  if (tid == 0) {
    a.ws.gt1[r.row * a.ws.P + p] = gtot;
    s_base = etot ? atomicAdd(&a.ws.meta[r.row].m, etot) : 0;
  }
  __syncthreads();
  if (ne) {
    unsigned long long *cl = a.ws.cand + r.row * a.ws.ldk + s_base + eoff;
    int o = 0;
#pragma unroll
    for (int i = 0; i < kPT; ++i) {
      if (key[i] != 0u && (key[i] >> (32 - kD1)) == b1) cl[o++] = composite(key[i], key_pos(j0, i));
    }
  }
}

// Bin of an nb-bin histogram (nb <= kBins2, highest bin = largest values)
// holding the want-th largest element: s_res = {bin, rank inside it, count}.
__device__ __forceinline__ void find_bin_row(const unsigned *hist, int nb, int want, int *s_wave,
                                             int *s_res) {
  const int t = threadIdx.x;
  constexpr int BPT = kBins2 / kRT;
  const int top = nb - 1 - BPT * t;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) cnt += (top - i >= 0) ? (int)hist[top - i] : 0;
  int total;
  const int above = block_exscan<kRW>(cnt, s_wave, &total);
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

// ---------------------------------------------------------- 5. threshold
__global__ __launch_bounds__(kRT) void threshold_kernel(SelectLaunch a) {
  __shared__ unsigned hist[kBins2];
  __shared__ int cnt[kSelMaxChunks];
  __shared__ int s_wave[kRW];
  __shared__ int s_res[3];
  RowGeo r;
  if (!row_geo(a, r)) return;
  const int tid = threadIdx.x;
  const int K = a.k;
  const int Pn = (r.span + kCH - 1) / kCH;
  const int b1 = a.ws.meta[r.row].b1;
  const int want1 = a.ws.meta[r.row].want1;
  const int m = (b1 != 0) ? a.ws.meta[r.row].m : 0;
  const unsigned long long *cl = a.ws.cand + r.row * a.ws.ldk;

  // Radix select of the want1-th largest composite among the m candidates.
  // Their top 12 bits all equal b1; digits of 11 bits cover bits 51..0.
  unsigned long long T = 0ull;
  if (m > 0) {
    unsigned long long prefix = (unsigned long long)b1;  // bits above the digit
    int top = 51, want = want1;
    for (;;) {
      const int lo_bit = max(top - kD2 + 1, 0);
      const int width = top - lo_bit + 1;
      const unsigned long long dmask = (1ull << width) - 1ull;
      for (int i = tid; i < (1 << width); i += kRT) hist[i] = 0u;
      if (tid == 0) {
        s_res[0] = 0;
        s_res[1] = 1;
        s_res[2] = 0;
      }
      __syncthreads();
      for (int i = tid; i < m; i += kRT) {
        const unsigned long long c = cl[i];
        if ((c >> (top + 1)) == prefix) atomicAdd(&hist[(c >> lo_bit) & dmask], 1u);
      }
      __syncthreads();
      find_bin_row(hist, 1 << width, want, s_wave, s_res);
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
  }

  // Winners per chunk: keys above the tie bin plus candidates >= T.
  for (int q = tid; q < Pn; q += kRT) cnt[q] = a.ws.gt1[r.row * a.ws.P + q];
  __syncthreads();
  for (int i = tid; i < m; i += kRT) {
    const unsigned long long c = cl[i];
    if (c >= T) {
      const int j = (int)(0xFFFFFFFFu - (uint32_t)(c & 0xFFFFFFFFull));
      atomicAdd(&cnt[j / kCH], 1);
    }
  }
  __syncthreads();
  // Output offset of every chunk (thread t scans chunks [t*CPT, t*CPT+CPT)).
  constexpr int CPT = kSelMaxChunks / kRT;
  int loc[CPT];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int q = tid * CPT + i;
    loc[i] = (q < Pn) ? cnt[q] : 0;
    sum += loc[i];
  }
  int total;
  int off = block_exscan<kRW>(sum, s_wave, &total);
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int q = tid * CPT + i;
    if (q < Pn) a.ws.offs[r.row * a.ws.P + q] = off;
    off += loc[i];
  }
  if (tid == 0) {
    a.ws.meta[r.row].T = T;
    a.sel_count[r.row] = min(total, K);
  }
  int32_t *out = a.sel_idx + r.row * K;
  for (int i = total + tid; i < K; i += kRT) out[i] = -1;
}

// --------------------------------------------------------- 6. compaction
__global__ __launch_bounds__(kT) void compact_kernel(SelectLaunch a) {
  __shared__ int s_wave[kTW];
  RowGeo r;
  if (!row_geo(a, r)) return;
  const int p = blockIdx.x, j0 = p * kCH;
  if (j0 >= r.span) return;
  const int tid = threadIdx.x;
  const int K = a.k;
  const uint32_t b1 = (uint32_t)a.ws.meta[r.row].b1;
  const unsigned long long T = a.ws.meta[r.row].T;
  const int base = a.ws.offs[r.row * a.ws.P + p];
  uint32_t key[kPT];
  load_keys(a.ws.keys + r.row * a.ws.ldk, j0, key);
  bool win[kPT];
  int c0 = 0, c1 = 0;
#pragma unroll
  for (int i = 0; i < kPT; ++i) {
    const uint32_t d = key[i] >> (32 - kD1);
    win[i] = key[i] != 0u &&
             (d > b1 || (b1 != 0u && d == b1 && composite(key[i], key_pos(j0, i)) >= T));
    if (i < 4) c0 += win[i] ? 1 : 0;
    else c1 += win[i] ? 1 : 0;
  }
  // ascending order: the first half chunk (four keys per thread, in thread
  // order), then the second
  int t0, t1;
  int o0 = block_exscan<kTW>(c0, s_wave, &t0);
  int o1 = t0 + block_exscan<kTW>(c1, s_wave, &t1);
  int32_t *out = a.sel_idx + r.row * K + base;
#pragma unroll
  for (int i = 0; i < kPT; ++i) {
    if (win[i]) {
      int &o = (i < 4) ? o0 : o1;
      if (base + o < K) out[o] = key_pos(j0, i);
      ++o;
    }
  }
}

}  // namespace

hipError_t launch_select(const SelectLaunch &a, hipStream_t st) {
  const dim3 grid(a.ws.P, a.H, a.batch_n);
  const dim3 rgrid(1, a.H, a.batch_n);
  const bool fused = a.mode == 0;
  hipError_t e;
  if (fused) {
    hipLaunchKernelGGL(norm_sums_kernel, grid, dim3(kT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(prior_kernel<true>, grid, dim3(kT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(keys_kernel<true>, grid, dim3(kT), 0, st, a);
  } else {
    hipLaunchKernelGGL(prior_kernel<false>, grid, dim3(kT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(keys_kernel<false>, grid, dim3(kT), 0, st, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tie_kernel, grid, dim3(kT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(threshold_kernel, rgrid, dim3(kRT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(compact_kernel, grid, dim3(kT), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfi
