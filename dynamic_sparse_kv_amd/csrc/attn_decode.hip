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
#include "sfi_internal.hpp"

namespace sfi {
namespace {

enum { MODE_SLOW = 0, MODE_FAST = 1 };
constexpr int kThreads = 256;
constexpr int kMaxFastChunk = 1024;

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
  float *key_norm;
  int ld;
  const int32_t *sel_idx;
  const int32_t *sel_count;
  int sel_heads, sel_k, n_sink, window;
  float qscale;  // log2(e) / sqrt(d)
};

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

template <int D, int G, bool PAGED, int MODE, bool EVID>
__global__ __launch_bounds__(kThreads) void partial_kernel(PartialArgs a) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPB = kThreads / LPR; // rows per workgroup instruction
  constexpr int U = 4;                // rows in flight per lane group
  constexpr int NW = kThreads / 64;

  __shared__ int s_idx[MODE == MODE_FAST ? kMaxFastChunk : 1];
  __shared__ float s_m[NW][G], s_z[NW][G];
  __shared__ float s_acc[NW][G][D];

  const int b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (b < 0) return;
  const int g = blockIdx.y;
  const int split = blockIdx.x;
  const int n = clamp_len(a.seq_len, b, a.max_len);
  const int tid = threadIdx.x;

  int L = n;
  FastList fl;
  if constexpr (MODE == MODE_FAST) {
    fl = fast_list(a.sel_idx, a.sel_count, a.sel_heads, a.sel_k, a.n_sink, a.window, b, g, n);
    L = fl.length();
  }
  const int p0 = split * a.chunk;
  if (p0 >= L) return;
  const int p1 = min(L, p0 + a.chunk);

  if constexpr (MODE == MODE_FAST) {
    for (int p = p0 + tid; p < p1; p += kThreads) {
      int j;
      if (p < fl.ns) {
        j = p;
      } else if (p < fl.ns + fl.nw) {
        j = fl.w0 + (p - fl.ns);
      } else {
        j = fl.sel[p - fl.ns - fl.nw];
        if (j < a.n_sink || j >= fl.w0) j = -1;  // padding, sink or now in window
      }
      s_idx[p - p0] = j;
    }
    __syncthreads();
  }

  const int sub = tid % LPR;
  const int rg = tid / LPR;

  uint32_t qv[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = ldg16(a.q + ((size_t)b * a.Hq + g * G + h) * D + sub * 8);
    qv[h][0] = t.x; qv[h][1] = t.y; qv[h][2] = t.z; qv[h][3] = t.w;
  }

  float m[G], Z[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    Z[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const size_t lrow = (size_t)(b * a.kv.Hkv + g);

  for (int base = p0 + rg; base < p1; base += RPB * U) {
    uint4 kr[U], vr[U];
    int jr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + u * RPB;
      int j = -1;
      if (p < p1) j = (MODE == MODE_FAST) ? s_idx[p - p0] : p;
      jr[u] = j;
      if (j >= 0) {
        const size_t off = kv_row<D, PAGED>(a.kv, b, g, j) + sub * 8;
        kr[u] = ldg16(a.kv.k + off);
        vr[u] = ldg16(a.kv.v + off);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = kr[u];
      }
    }

    float l[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = dot2_bf16(qv[h][0], kr[u].x, 0.f);
        s = dot2_bf16(qv[h][1], kr[u].y, s);
        s = dot2_bf16(qv[h][2], kr[u].z, s);
        s = dot2_bf16(qv[h][3], kr[u].w, s);
        s = group_sum<LPR>(s);
        l[u][h] = (jr[u] >= 0) ? s * a.qscale : -INFINITY;
      }
    }

    if constexpr (EVID) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float nn = dot2_bf16(kr[u].x, kr[u].x, 0.f);
        nn = dot2_bf16(kr[u].y, kr[u].y, nn);
        nn = dot2_bf16(kr[u].z, kr[u].z, nn);
        nn = dot2_bf16(kr[u].w, kr[u].w, nn);
        nn = group_sum<LPR>(nn);
        const int j = jr[u];
        if (j >= 0) {
          if (sub < G) {
            float v = l[u][0];
#pragma unroll
            for (int h = 1; h < G; ++h) v = (sub == h) ? l[u][h] : v;
            a.logits[(lrow * a.lld + j) * G + sub] = v;
          }
          if (sub == 0 && a.key_norm) a.key_norm[lrow * a.ld + j] = sqrtf(nn);
        }
      }
    }

    float vf[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vf[u][0] = bf_lo(vr[u].x); vf[u][1] = bf_hi(vr[u].x);
      vf[u][2] = bf_lo(vr[u].y); vf[u][3] = bf_hi(vr[u].y);
      vf[u][4] = bf_lo(vr[u].z); vf[u][5] = bf_hi(vr[u].z);
      vf[u][6] = bf_lo(vr[u].w); vf[u][7] = bf_hi(vr[u].w);
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = l[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, l[u][h]);
      const float mn = fmaxf(m[h], mx);
      const float sc = exp2f(m[h] - mn);
      m[h] = mn;
      Z[h] *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= sc;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pu = exp2f(l[u][h] - mn);
        Z[h] += pu;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pu, vf[u][e], acc[h][e]);
      }
    }
  }

  // Merge the lane groups of each wave (they hold the same dimensions).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float zo = __shfl_xor(Z[h], off);
      const float mn = fmaxf(m[h], mo);
      const float s1 = exp2f(m[h] - mn), s2 = exp2f(mo - mn);
      Z[h] = Z[h] * s1 + zo * s2;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * s1 + __shfl_xor(acc[h][e], off) * s2;
      m[h] = mn;
    }
  }

  const int lane = tid & 63, wv = tid >> 6;
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wv][h][lane * 8 + e] = acc[h][e];
      if (lane == 0) {
        s_m[wv][h] = m[h];
        s_z[wv][h] = Z[h];
      }
    }
  }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D, e = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float o = 0.f, z = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = exp2f(s_m[w][h] - M);
      o = fmaf(s_acc[w][h][e], sc, o);
      z = fmaf(s_z[w][h], sc, z);
    }
    const size_t slot = ((size_t)b * a.Hq + g * G + h) * a.stride + split;
    a.part_o[slot * D + e] = o;
    if (e == 0) {
      a.part_ml[slot * 2 + 0] = M;
      a.part_ml[slot * 2 + 1] = z;
    }
  }
}

struct FinalArgs {
  int B, max_len;
  const int32_t *seq_len;
  const int32_t *batch_ids;
  int Hq, Hkv;
  int chunk, stride;
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
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// grid.x = G combine blocks (one per query head of the group) followed, for
// slow steps with evidence, by one block per kEvidChunk keys.
template <int D, int G, int MODE, bool EVID>
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalArgs a) {
  constexpr int NW = kThreads / 64;
  constexpr int PARTS = kThreads / D;
  __shared__ float red[NW][G];
  __shared__ float s_part[PARTS][D];

  const int b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (b < 0) return;
  const int g = blockIdx.y;
  const int x = blockIdx.x;
  const int n = clamp_len(a.seq_len, b, a.max_len);
  int L = n;
  if constexpr (MODE == MODE_FAST) {
    L = fast_list(a.sel_idx, a.sel_count, a.sel_heads, a.sel_k, a.n_sink, a.window, b, g, n)
            .length();
  }
  const bool comb = x < G;
  if (!comb && (x - G) * kEvidChunk >= n) return;
  const int S = (L + a.chunk - 1) / a.chunk;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t hbase = (size_t)b * a.Hq + (size_t)g * G;

  // Global running max and normaliser of every head of the group.
  float M[G], Zs[G];
  {
    float ml[G];
#pragma unroll
    for (int h = 0; h < G; ++h) ml[h] = kNegBig;
    for (int s = tid; s < S; s += kThreads) {
#pragma unroll
      for (int h = 0; h < G; ++h) ml[h] = fmaxf(ml[h], a.part_ml[((hbase + h) * a.stride + s) * 2]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      ml[h] = wave_max(ml[h]);
      if (lane == 0) red[wv][h] = ml[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float v = red[0][h];
#pragma unroll
      for (int w = 1; w < NW; ++w) v = fmaxf(v, red[w][h]);
      M[h] = v;
    }
    __syncthreads();
    float zl[G];
#pragma unroll
    for (int h = 0; h < G; ++h) zl[h] = 0.f;
    for (int s = tid; s < S; s += kThreads) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float *ml2 = a.part_ml + ((hbase + h) * a.stride + s) * 2;
        zl[h] = fmaf(ml2[1], exp2f(ml2[0] - M[h]), zl[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      zl[h] = wave_sum(zl[h]);
      if (lane == 0) red[wv][h] = zl[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += red[w][h];
      Zs[h] = v;
    }
  }

  if (comb) {
    float Mh = M[0], Zh = Zs[0];
#pragma unroll
    for (int h = 1; h < G; ++h) {
      Mh = (x == h) ? M[h] : Mh;
      Zh = (x == h) ? Zs[h] : Zh;
    }
    const size_t row = hbase + x;
    const int e = tid % D, part = tid / D;
    float o = 0.f;
    for (int s = part; s < S; s += PARTS) {
      const float w = exp2f(a.part_ml[(row * a.stride + s) * 2] - Mh);
      o = fmaf(w, a.part_o[(row * a.stride + s) * D + e], o);
    }
    s_part[part][e] = o;
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int p = 1; p < PARTS; ++p) o += s_part[p][e];
      a.out[row * D + e] = (Zh > 0.f) ? o / Zh : 0.f;
    }
    return;
  }

  if constexpr (EVID) {
    float rz[G];
#pragma unroll
    for (int h = 0; h < G; ++h) rz[h] = 1.0f / ((float)G * Zs[h]);
    const size_t lrow = (size_t)b * a.Hkv + g;
    const int j0 = (x - G) * kEvidChunk;
    const int j1 = min(n, j0 + kEvidChunk);
    for (int j = j0 + tid; j < j1; j += kThreads) {
      const float *lp = a.logits + (lrow * a.lld + j) * G;
      float f = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) f = fmaf(exp2f(lp[h] - M[h]), rz[h], f);
      a.evidence[lrow * a.ld + j] = f;
    }
  }
}

template <int D, int G, bool PAGED>
hipError_t slow_t(const AttnLaunch &a, hipStream_t st) {
  PartialArgs p{};
  p.B = a.B; p.max_len = a.max_len;
  p.kv = a.kv; p.seq_len = a.seq_len; p.batch_ids = a.batch_ids; p.q = a.q; p.Hq = a.Hq;
  p.chunk = a.plan.chunk; p.stride = a.plan.stride; p.part_o = a.part_o; p.part_ml = a.part_ml;
  p.logits = a.logits; p.lld = a.lld; p.key_norm = a.key_norm; p.ld = a.ld;
  p.qscale = kLog2e / sqrtf((float)D);
  const bool side = a.evidence != nullptr || a.key_norm != nullptr;
  dim3 grid(a.plan.splits, a.Hkv, a.batch_n);
  if (side)
    hipLaunchKernelGGL((partial_kernel<D, G, PAGED, MODE_SLOW, true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((partial_kernel<D, G, PAGED, MODE_SLOW, false>), grid, dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  FinalArgs f{};
  f.B = a.B; f.max_len = a.max_len;
  f.seq_len = a.seq_len; f.batch_ids = a.batch_ids; f.Hq = a.Hq; f.Hkv = a.Hkv;
  f.chunk = a.plan.chunk; f.stride = a.plan.stride; f.part_o = a.part_o; f.part_ml = a.part_ml;
  f.out = a.out; f.logits = a.logits; f.lld = a.lld; f.evidence = a.evidence; f.ld = a.ld;
  const int kv_max = a.plan.splits * a.plan.chunk;
  const int nev = a.evidence ? (kv_max + kEvidChunk - 1) / kEvidChunk : 0;
  dim3 g2(G + nev, a.Hkv, a.batch_n);
  if (a.evidence)
    hipLaunchKernelGGL((finalize_kernel<D, G, MODE_SLOW, true>), g2, dim3(kThreads), 0, st, f);
  else
    hipLaunchKernelGGL((finalize_kernel<D, G, MODE_SLOW, false>), g2, dim3(kThreads), 0, st, f);
  return hipGetLastError();
}

template <int D, int G, bool PAGED>
hipError_t fast_t(const AttnLaunch &a, hipStream_t st) {
  PartialArgs p{};
  p.B = a.B; p.max_len = a.max_len;
  p.kv = a.kv; p.seq_len = a.seq_len; p.batch_ids = a.batch_ids; p.q = a.q; p.Hq = a.Hq;
  p.chunk = a.plan.chunk; p.stride = a.plan.stride; p.part_o = a.part_o; p.part_ml = a.part_ml;
  p.sel_idx = a.sel_idx; p.sel_count = a.sel_count; p.sel_heads = a.sel_heads; p.sel_k = a.sel_k;
  p.n_sink = a.n_sink; p.window = a.window;
  p.qscale = kLog2e / sqrtf((float)D);
  dim3 grid(a.plan.splits, a.Hkv, a.batch_n);
  hipLaunchKernelGGL((partial_kernel<D, G, PAGED, MODE_FAST, false>), grid, dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FinalArgs f{};
  f.B = a.B; f.max_len = a.max_len;
  f.seq_len = a.seq_len; f.batch_ids = a.batch_ids; f.Hq = a.Hq; f.Hkv = a.Hkv;
  f.chunk = a.plan.chunk; f.stride = a.plan.stride; f.part_o = a.part_o; f.part_ml = a.part_ml;
  f.out = a.out; f.sel_idx = a.sel_idx; f.sel_count = a.sel_count; f.sel_heads = a.sel_heads;
  f.sel_k = a.sel_k; f.n_sink = a.n_sink; f.window = a.window;
  dim3 g2(G, a.Hkv, a.batch_n);
  hipLaunchKernelGGL((finalize_kernel<D, G, MODE_FAST, false>), g2, dim3(kThreads), 0, st, f);
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

int slow_chunk_for(int batch_n, int Hkv, int max_seq_len) {
  // Aim at >= 2048 workgroups (8 per CU) with chunks of 256..8192 rows.
  const long long rows = (long long)batch_n * Hkv * max_seq_len;
  int chunk = kMinSlowChunk;
  while (chunk < kMaxSlowChunk && rows / (2LL * chunk) >= 2048) chunk *= 2;
  return chunk;
}

hipError_t launch_slow(const AttnLaunch &a, hipStream_t st) { SFI_DISPATCH(slow_t, a, st); }
hipError_t launch_fast(const AttnLaunch &a, hipStream_t st) {
  if (a.plan.chunk > kMaxFastChunk) return hipErrorInvalidValue;
  SFI_DISPATCH(fast_t, a, st);
}

}  // namespace sfi
