// Training-free selector on gfx950.
//
// Slow-Fast Inference (technical summary section 3.B; Korean summary section
// 2.B): the slow step's evidence f is fused with a prior r built from cache
// statistics (key norms and positions) by the reverse-KL objective whose
// minimiser is the mixture s = (1 - lambda) f + lambda r; the Top-K of s over
// the selectable keys becomes the next selected memory.  Vegas (section 2.A)
// ranks aggregated verify logits the same way, with one list per sequence.
//
// One 1024-thread workgroup per (sequence, head row) does the whole job in a
// single launch.  A block of 40960 keys is 10 slabs of 4096; thread t owns
// keys 4t..4t+3 of every slab (one coalesced 16-byte access per slab).  When
// the row fits one block (contexts up to 40K) the values never leave
// registers between phases:
//   1. mean, then population variance of the key norms (two passes, fp32
//      per thread, fp64 across the workgroup);
//   2. prior weights w_j = exp(-c z_j)(1 + exp(-(t-j)/tau)) and their sum;
//   3. s_j = (1-lambda) f_j + lambda w_j / sum(w), turned into an
//      order-preserving 32-bit key, with the min and max key of the
//      candidates;
//   4. radix select of the k-th largest key: 12-bit LDS histograms starting
//      at the highest bit where min and max differ (the bits above are
//      common to every candidate, so the first digit already spreads the
//      keys), stopping as soon as the threshold bin is taken whole;
//   5. ordered compaction through LDS bitmaps: winners (and, when the
//      threshold key is tied, the lowest-index ties) are marked, one scan of
//      per-word popcounts places every word, indices come out ascending.
// Longer rows stream their blocks from L2 in every phase instead.
#include "sfi_internal.hpp"

namespace sfi {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSlabs = 10;                        // slabs per block
constexpr int kSlab = kSelThreads * 4;            // 4096 keys per slab
constexpr int kVPT = kSlabs * 4;                  // values per thread per block
constexpr int kBlock = kSelThreads * kVPT;        // 40960 keys
constexpr int kDigit = 12;                        // radix digit width
constexpr int kBins = 1 << kDigit;
constexpr int kWords = kBlock / 32;               // bitmap words per block

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Sum over the workgroup in a fixed order (deterministic).
__device__ __forceinline__ double block_sum_d(double x, double *s_red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  x = wave_sum_d(x);
  if (lane == 0) s_red[wv] = x;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) t += s_red[w];
  __syncthreads();
  return t;
}

// Workgroup min and max of a key.
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, uint32_t *s_u,
                                             uint32_t *out_mn, uint32_t *out_mx) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  }
  if (lane == 0) {
    s_u[wv] = mn;
    s_u[kSelWaves + wv] = mx;
  }
  __syncthreads();
  uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    a = min(a, s_u[w]);
    b = max(b, s_u[kSelWaves + w]);
  }
  __syncthreads();
  *out_mn = a;
  *out_mx = b;
}

// Population count as a signed int (HIP's __popc returns unsigned, which would
// turn differences of counts into wrapped unsigned values).
__device__ __forceinline__ int popc32(uint32_t x) { return (int)__popc(x); }

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
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

// Bin of a histogram (nb <= kBins bins; highest bin = largest keys) that
// holds the want-th largest element: s_res = {bin, rank inside, bin count}.
__device__ __forceinline__ void find_bin(const unsigned *hist, int nb, int want, int *s_wave,
                                         int *s_res) {
  const int t = threadIdx.x;
  if (t == 0) {
    s_res[0] = 0;
    s_res[1] = 1;
    s_res[2] = 0;
  }
  const int hi = nb - 1 - 4 * t;
  int cnt = 0;
  if (hi >= 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt += (hi - i >= 0) ? (int)hist[hi - i] : 0;
  }
  int total;
  const int above = block_exscan(cnt, s_wave, &total);
  if (hi >= 0 && above < want && want <= above + cnt) {
    int acc = above;
    for (int i = 0; i < 4 && hi - i >= 0; ++i) {
      const int c = (int)hist[hi - i];
      if (acc + c >= want) {
        s_res[0] = hi - i;
        s_res[1] = want - acc;
        s_res[2] = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

template <bool FUSED>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectLaunch a) {
  __shared__ unsigned hist[kBins];
  __shared__ uint32_t bm_sel[kWords];  // per-block bitmap of winners
  __shared__ uint32_t bm_eq[kWords];   // per-block bitmap of threshold ties
  __shared__ int s_wave[kSelWaves];
  __shared__ uint32_t s_u[2 * kSelWaves];
  __shared__ double s_red[kSelWaves];
  __shared__ int s_res[3];

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
  const bool take_all = ncand <= K;
  int32_t *out = a.sel_idx + row * K;

  // keys [0, span) are visited (uniform: it steers the slab-level branches)
  const int span = __builtin_amdgcn_readfirstlane(FUSED ? n : hi);
  const int NB = (span + kBlock - 1) / kBlock;
  const bool resident = NB <= 1;
  const float *score = a.score + row * a.ld;
  float *sb = FUSED ? a.sbuf + row * a.sld : nullptr;
  const float *src = FUSED ? (const float *)sb : score;  // ranked values when streaming

  // Value i of this thread in block blk is key blk*kBlock + (i/4)*kSlab + 4*tid + i%4.
  auto key_of = [&](int blk, int i) { return blk * kBlock + (i >> 2) * kSlab + 4 * tid + (i & 3); };
  // u[] holds the raw float bits of the current block until make_keys turns
  // them into order-preserving keys in place.
  uint32_t u[kVPT];
  // Slab-level cases are uniform across the workgroup: a whole slab in range
  // takes one 16-byte load per thread, a slab past the end takes none, and
  // only the slab that holds the end of the row uses clamped scalar loads.
  // No load sits behind a per-lane branch, so all slabs' loads are in flight
  // together (a per-lane branch makes the compiler drain them one by one).
  auto load4 = [&](const float *p, int slab0, bool vec, float (&x)[4]) {
    const int j = slab0 + 4 * tid;
    if (vec && slab0 + kSlab <= span) {
      const float4 t = *reinterpret_cast<const float4 *>(p + j);
      x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
    } else if (slab0 >= span) {
      x[0] = x[1] = x[2] = x[3] = 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = p[min(j + e, span - 1)];
        x[e] = (j + e < span) ? t : 0.f;
      }
    }
  };
  auto load = [&](const float *p, int blk, bool vec) {
#pragma unroll
    for (int sl = 0; sl < kSlabs; ++sl) {
      float x[4];
      load4(p, blk * kBlock + sl * kSlab, vec, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * sl + e] = __float_as_uint(x[e]);
    }
  };
  auto store = [&](float *p, int blk, bool vec) {
#pragma unroll
    for (int sl = 0; sl < kSlabs; ++sl) {
      const int j = blk * kBlock + sl * kSlab + 4 * tid;
      if (vec && j + 4 <= span) {
        *reinterpret_cast<float4 *>(p + j) =
            make_float4(__uint_as_float(u[4 * sl + 0]), __uint_as_float(u[4 * sl + 1]),
                        __uint_as_float(u[4 * sl + 2]), __uint_as_float(u[4 * sl + 3]));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j + e < span) p[j + e] = __uint_as_float(u[4 * sl + e]);
      }
    }
  };
  // 16-byte accesses need 16-byte aligned rows.
  const float *nu = FUSED ? a.key_norm + row * a.ld : nullptr;
  const bool vsc = ((reinterpret_cast<uintptr_t>(score) | reinterpret_cast<uintptr_t>(nu)) & 15u) == 0;
  const bool vsb = FUSED ? ((reinterpret_cast<uintptr_t>(sb) & 15u) == 0) : vsc;
  const bool vsrc = FUSED ? vsb : vsc;

  // Keys of non-candidates (j outside [lo, hi)) are set to 0.  Every finite
  // or infinite score maps to a key >= 0x007FFFFF, and the radix digits never
  // put such a key in the bin of 0, so 0 marks "not a candidate" exactly.
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;  // candidate key range of this thread
  auto make_keys = [&](int blk) {
#pragma unroll
    for (int sl = 0; sl < kSlabs; ++sl) {
      const int j0 = blk * kBlock + sl * kSlab + 4 * tid;
      const bool all_in = j0 >= lo && j0 + 3 < hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * sl + e;
        const bool in = all_in || (j0 + e >= lo && j0 + e < hi);
        u[i] = in ? float_key(__uint_as_float(u[i])) : 0u;
      }
    }
  };
  auto range_add = [&]() {
#pragma unroll
    for (int i = 0; i < kVPT; ++i) {
      kmin = min(kmin, u[i] ? u[i] : 0xFFFFFFFFu);
      kmax = max(kmax, u[i]);
    }
  };
  // Keys of block blk: already in registers for a resident row, else reloaded.
  auto block_keys = [&](int blk) {
    if (!resident) {
      load(src, blk, vsrc);
      make_keys(blk);
    }
  };

  if constexpr (FUSED) {
    // Mean and population variance in two passes (per-thread fp32 partials,
    // fp64 across the workgroup), so no large-number cancellation.
    float s1f = 0.f;
    for (int blk = 0; blk < NB; ++blk) {
      if (!resident || blk == 0) load(nu, blk, vsc);
#pragma unroll
      for (int i = 0; i < kVPT; ++i) s1f += __uint_as_float(u[i]);
    }
    const double mu = n > 0 ? block_sum_d((double)s1f, s_red) / n : 0.0;
    const float muf = (float)mu;
    float s2f = 0.f;
    for (int blk = 0; blk < NB; ++blk) {
      if (!resident) load(nu, blk, vsc);
#pragma unroll
      for (int i = 0; i < kVPT; ++i) {
        const float dv = (key_of(blk, i) < n) ? __uint_as_float(u[i]) - muf : 0.f;
        s2f = fmaf(dv, dv, s2f);
      }
    }
    const double var = n > 0 ? block_sum_d((double)s2f, s_red) / n : 0.0;
    const double sd = sqrt(var);
    const float isd = sd > 0.0 ? (float)(1.0 / sd) : 0.0f;
    const float tq = (float)(n - 1);
    // w_j = exp(-c z_j) (1 + exp(-(t - j)/tau)) evaluated as powers of two.
    const float cz = -a.norm_coef * isd * kLog2e;
    const float ct = kLog2e / a.pos_tau;
    double sw = 0.0;
    for (int blk = 0; blk < NB; ++blk) {
      if (!resident) load(nu, blk, vsc);
      float swf = 0.f;
#pragma unroll
      for (int i = 0; i < kVPT; ++i) {
        const int j = key_of(blk, i);
        const float w = (j < n) ? exp2f(cz * (__uint_as_float(u[i]) - muf)) * (1.0f + exp2f(((float)j - tq) * ct)) : 0.f;
        u[i] = __float_as_uint(w);
        swf += w;
      }
      sw += (double)swf;
      if (!resident) store(sb, blk, vsb);
    }
    const double W = block_sum_d(sw, s_red);
    const float cf = 1.0f - a.lambda;
    const float cr = W > 0.0 ? (float)((double)a.lambda / W) : 0.f;
    for (int blk = 0; blk < NB; ++blk) {
      if (!resident) load(sb, blk, vsb);
#pragma unroll
      for (int sl = 0; sl < kSlabs; ++sl) {
        float f4[4];
        load4(score, blk * kBlock + sl * kSlab, vsc, f4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          u[4 * sl + e] = __float_as_uint(fmaf(cf, f4[e], cr * __uint_as_float(u[4 * sl + e])));
      }
      if (!resident || a.store_s) store(sb, blk, vsb);
      make_keys(blk);
      range_add();
    }
  } else {
    for (int blk = 0; blk < NB; ++blk) {
      load(score, blk, vsc);
      make_keys(blk);
      range_add();
    }
  }
  block_minmax(kmin, kmax, s_u, &kmin, &kmax);

  // Radix select.  Selected = keys whose bits at and above `lvl` exceed `thr`,
  // plus the first take_eq (by index) of those equal to it.
  uint32_t thr = 0u;
  int lvl = 0;
  int take_eq = 0;
  int eq_total = 0;  // candidates whose (key >> lvl) equals thr
  if (!take_all) {
    const uint32_t diff = kmin ^ kmax;
    if (diff == 0u) {  // every candidate has the same key
      thr = kmax;
      take_eq = K;
      eq_total = ncand;
    } else {
      int top = 31 - __builtin_clz(diff);                       // highest differing bit
      uint32_t prefix = (top >= 31) ? 0u : (kmax >> (top + 1));  // common bits above it
      int want = K;
      for (;;) {
        const int lo_bit = max(top - kDigit + 1, 0);
        const int width = top - lo_bit + 1;
        const uint32_t dmask = (1u << width) - 1u;
        for (int i = tid; i < (1 << width); i += kSelThreads) hist[i] = 0u;
        __syncthreads();
        const int sh_up = top + 1;
        for (int blk = 0; blk < NB; ++blk) {
          block_keys(blk);
#pragma unroll
          for (int i = 0; i < kVPT; ++i) {
            const uint32_t up = (sh_up >= 32) ? 0u : (u[i] >> sh_up);
            if (u[i] && up == prefix) atomicAdd(&hist[(u[i] >> lo_bit) & dmask], 1u);
          }
        }
        __syncthreads();
        find_bin(hist, 1 << width, want, s_wave, s_res);
        const uint32_t bin = (uint32_t)s_res[0];
        want = s_res[1];
        const int cnt = s_res[2];
        __syncthreads();
        prefix = (width >= 32) ? bin : ((prefix << width) | bin);
        if (lo_bit == 0 || want == cnt) {  // exact key reached, or the whole bin is taken
          thr = prefix;
          lvl = lo_bit;
          take_eq = want;
          eq_total = cnt;
          break;
        }
        top = lo_bit - 1;
      }
    }
  }

  // Ordered compaction through per-block bitmaps: winners are marked in
  // bm_sel (ties at the threshold in bm_eq, of which the first take_eq by
  // index are kept), then one scan of per-word popcounts gives every word
  // its output offset, so indices come out ascending.
  const bool ge_mode = take_all || take_eq == eq_total;  // the whole tie bin is taken
  const bool inc = (tid * 2) < kWords;
  int carry_eq = 0, carry_sel = 0;
  for (int blk = 0; blk < NB; ++blk) {
    for (int w = tid; w < kWords; w += kSelThreads) {
      bm_sel[w] = 0u;
      bm_eq[w] = 0u;
    }
    __syncthreads();
    block_keys(blk);
#pragma unroll
    for (int sl = 0; sl < kSlabs; ++sl) {
      uint32_t ngt = 0u, neq = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * sl + e;
        const bool in = u[i] != 0u;
        const uint32_t kk = u[i] >> lvl;
        const bool gt = in && (take_all || (ge_mode ? kk >= thr : kk > thr));
        const bool eq = in && !ge_mode && kk == thr;
        ngt |= (gt ? 1u : 0u) << e;
        neq |= (eq ? 1u : 0u) << e;
      }
      const int word = sl * (kSlab / 32) + (tid >> 3);
      const int sh = (tid & 7) * 4;
      if (ngt) atomicOr(&bm_sel[word], ngt << sh);
      if (neq) atomicOr(&bm_eq[word], neq << sh);
    }
    __syncthreads();
    if (!ge_mode) {
      const uint32_t e0 = inc ? bm_eq[2 * tid] : 0u, e1 = inc ? bm_eq[2 * tid + 1] : 0u;
      int tot;
      const int before = carry_eq + block_exscan(popc32(e0) + popc32(e1), s_wave, &tot);
      if (inc) {
        // keep the lowest `m` set bits of each tie word
        int m0 = min(max(take_eq - before, 0), popc32(e0));
        uint32_t keep0 = 0u, w0 = e0;
        for (; m0 > 0; --m0) { const uint32_t lb = w0 & (0u - w0); keep0 |= lb; w0 ^= lb; }
        int m1 = min(max(take_eq - before - popc32(e0), 0), popc32(e1));
        uint32_t keep1 = 0u, w1 = e1;
        for (; m1 > 0; --m1) { const uint32_t lb = w1 & (0u - w1); keep1 |= lb; w1 ^= lb; }
        bm_sel[2 * tid] |= keep0;
        bm_sel[2 * tid + 1] |= keep1;
      }
      carry_eq += tot;
      __syncthreads();
    }
    const uint32_t s0 = inc ? bm_sel[2 * tid] : 0u, s1 = inc ? bm_sel[2 * tid + 1] : 0u;
    int tot;
    int pos = carry_sel + block_exscan(popc32(s0) + popc32(s1), s_wave, &tot);
    if (inc) {
      const int base = blk * kBlock;
      uint32_t w = s0;
      while (w) {
        const int bit = __ffs(w) - 1;
        w &= w - 1u;
        // word 2t holds keys of slab (2t / 128), lanes 4*(t' ...): decode its key index
        const int wd = 2 * tid;
        const int j = base + (wd / (kSlab / 32)) * kSlab + (wd % (kSlab / 32)) * 32 + bit;
        if (pos < K) out[pos] = j;
        ++pos;
      }
      w = s1;
      while (w) {
        const int bit = __ffs(w) - 1;
        w &= w - 1u;
        const int wd = 2 * tid + 1;
        const int j = base + (wd / (kSlab / 32)) * kSlab + (wd % (kSlab / 32)) * 32 + bit;
        if (pos < K) out[pos] = j;
        ++pos;
      }
    }
    carry_sel += tot;
    __syncthreads();
  }
  for (int i = carry_sel + tid; i < K; i += kSelThreads) out[i] = -1;
  if (tid == 0) a.sel_count[row] = min(carry_sel, K);
}

}  // namespace

hipError_t launch_select(const SelectLaunch &a, hipStream_t st) {
  if (a.mode == 0)
    hipLaunchKernelGGL(select_kernel<true>, dim3(a.H, a.batch_n), dim3(kSelThreads), 0, st, a);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3(a.H, a.batch_n), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sfi
