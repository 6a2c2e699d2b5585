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

namespace sfi {
namespace {

#ifndef SFI_DECODE_U
#define SFI_DECODE_U 2
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
  // 8 lanes per row halves the cross-lane reduction and softmax work per row
  // compared with 16; wide groups (G*D > 640) use 16 to bound accumulators.
  constexpr int LPR = (G * D > 640) ? 16 : 8;  // lanes per row
  constexpr int DPL = D / LPR;         // dims per lane (8 or 16)
  constexpr int NV = DPL / 8;          // 16-byte slices per row per lane
  constexpr int RPB = kThreads / LPR;  // rows per workgroup instruction
  constexpr int U = SFI_DECODE_U;      // rows per lane group per pipeline stage
  constexpr int NW = kThreads / 64;
  // Lazy rescaling: the running reference m only moves when a logit exceeds
  // it by more than kSlack (log2 units), so p = 2^(l - m) stays <= 2^kSlack.
  constexpr float kSlack = 8.0f;

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

  const int sub = tid % LPR;
  const int rg = tid / LPR;

  uint32_t qv[G][4 * NV];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int c = 0; c < NV; ++c) {
      const uint4 t = ldg16(a.q + ((size_t)b * a.Hq + g * G + h) * D + sub * DPL + 8 * c);
      qv[h][4 * c + 0] = t.x; qv[h][4 * c + 1] = t.y; qv[h][4 * c + 2] = t.z; qv[h][4 * c + 3] = t.w;
    }
  }

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


  float m[G], Z[G], acc[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    Z[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
  }

  const size_t lrow = (size_t)(b * a.kv.Hkv + g);

  // One pipeline stage: U rows per lane group, K and V slices of DPL dims.
  struct Stage {
    uint4 k[U][NV], v[U][NV];
    int j[U];
  };
  auto load_stage = [&](Stage &st, int base) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = base + u * RPB;
      int j = -1;
      if (p < p1) j = (MODE == MODE_FAST) ? s_idx[p - p0] : p;
      st.j[u] = j;
      if (j >= 0) {
        const size_t off = kv_row<D, PAGED>(a.kv, b, g, j) + sub * DPL;
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          st.k[u][c] = ldg16(a.kv.k + off + 8 * c);
          st.v[u][c] = ldg16(a.kv.v + off + 8 * c);
        }
      } else {
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          st.k[u][c] = make_uint4(0, 0, 0, 0);
          st.v[u][c] = st.k[u][c];
        }
      }
    }
  };
  auto consume = [&](const Stage &st) {
    float l[U][G];
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
        l[u][h] = (st.j[u] >= 0) ? sdot * a.qscale : -INFINITY;
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
        const int j = st.j[u];
        if (j >= 0) {
          if (sub < G) {
            float v = l[u][0];
#pragma unroll
            for (int h = 1; h < G; ++h) v = (sub == h) ? l[u][h] : v;
            a.logits[(lrow * a.lld + j) * G + sub] = v;
          }
          if (sub == G % LPR && a.key_norm) a.key_norm[lrow * a.ld + j] = sqrtf(nn);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = l[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, l[u][h]);
      const bool need = mx > m[h] + kSlack;
      if (__any(need)) {
        const float mn = need ? mx : m[h];
        const float sc = exp2f(m[h] - mn);
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
        pu[h] = exp2f(l[u][h] - m[h]);
        Z[h] += pu[h];
      }
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        const uint32_t w4[4] = {st.v[u][c].x, st.v[u][c].y, st.v[u][c].z, st.v[u][c].w};
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
  Stage sa, sb;
  load_stage(sa, p0 + rg);
  for (int base = p0 + rg; base < p1; base += 2 * STEP) {
    load_stage(sb, base + STEP);
    consume(sa);
    load_stage(sa, base + 2 * STEP);
    consume(sb);
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
    auto xch = [&](float x) -> float {
      if constexpr (OFF == 8) return dpp_f32<0x128>(x);  // row_ror:8 == lane ^ 8 within a row
      else return __shfl_xor(x, OFF);
    };
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = xch(m[h]);
      const float zo = xch(Z[h]);
      const float mn = fmaxf(m[h], mo);
      const float s1 = exp2f(m[h] - mn), s2 = exp2f(mo - mn);
      Z[h] = Z[h] * s1 + zo * s2;
      m[h] = mn;
#pragma unroll
      for (int i = 0; i < HALF; ++i) {
        const float keep = bit ? acc[h][HALF + i] : acc[h][i];
        const float send = bit ? acc[h][i] : acc[h][HALF + i];
        acc[h][i] = keep * s1 + xch(send) * s2;
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
    for (int i = 0; i < KEPT; ++i) s_acc[wv][h][sub * DPL + dim_off + i] = acc[h][i];
    if (lane == 0) {
      s_m[wv][h] = m[h];
      s_z[wv][h] = Z[h];
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
  __shared__ float red[NW][G];

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
    // PARTS4 groups of D/4 threads; each thread merges 4 dims of every
    // PARTS4-th partial, four partials in flight at a time.
    constexpr int TPP = D / 4;
    constexpr int PARTS4 = kThreads / TPP;
    const size_t row = hbase + x;
    const int e4 = tid % TPP, part = tid / TPP;
    const float *pm = a.part_ml + row * a.stride * 2;
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o + row * a.stride * D) + e4;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = part;
    for (; s + 3 * PARTS4 < S; s += 4 * PARTS4) {
      float4 v[4];
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = po[(size_t)(s + i * PARTS4) * TPP];
        w[i] = pm[(s + i * PARTS4) * 2];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float wi = exp2f(w[i] - Mh);
        o.x = fmaf(wi, v[i].x, o.x);
        o.y = fmaf(wi, v[i].y, o.y);
        o.z = fmaf(wi, v[i].z, o.z);
        o.w = fmaf(wi, v[i].w, o.w);
      }
    }
    for (; s < S; s += PARTS4) {
      const float4 v = po[(size_t)s * TPP];
      const float wi = exp2f(pm[s * 2] - Mh);
      o.x = fmaf(wi, v.x, o.x);
      o.y = fmaf(wi, v.y, o.y);
      o.z = fmaf(wi, v.z, o.z);
      o.w = fmaf(wi, v.w, o.w);
    }
    __shared__ float4 s_o4[PARTS4][TPP];
    s_o4[part][e4] = o;
    __syncthreads();
    if (part == 0) {
#pragma unroll
      for (int p = 1; p < PARTS4; ++p) {
        const float4 t = s_o4[p][e4];
        o.x += t.x; o.y += t.y; o.z += t.z; o.w += t.w;
      }
      const float rz = (Zh > 0.f) ? 1.0f / Zh : 0.f;
      float4 r = make_float4(o.x * rz, o.y * rz, o.z * rz, o.w * rz);
      if (Zh <= 0.f) r = make_float4(0.f, 0.f, 0.f, 0.f);
      reinterpret_cast<float4 *>(a.out + row * D)[e4] = r;
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
    constexpr int PER = kEvidChunk / kThreads;
    float lg[PER][G];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = j0 + tid + i * kThreads;
      const float *lp = a.logits + (lrow * a.lld + (size_t)min(j, j1 - 1)) * G;
#pragma unroll
      for (int h = 0; h < G; ++h) lg[i][h] = lp[h];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = j0 + tid + i * kThreads;
      float f = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) f = fmaf(exp2f(lg[i][h] - M[h]), rz[h], f);
      if (j < j1) a.evidence[lrow * a.ld + j] = f;
    }
  }
}

// Resident workgroups of one kernel instance across the device (cached).
template <typename Kern>
int resident_slots(Kern kern) {
  static int slots[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (slots[dev] == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kThreads, 0) != hipSuccess || nb < 1) nb = 1;
    slots[dev] = nb * device_cu_count() * SFI_WAVES_OF_WG;
  }
  return slots[dev];
}

template <int D, int G, bool PAGED>
hipError_t slow_t(const AttnLaunch &a_in, hipStream_t st) {
  AttnLaunch a = a_in;
  const bool side = a.evidence != nullptr || a.key_norm != nullptr;
  {
    const int slots = side ? resident_slots(partial_kernel<D, G, PAGED, MODE_SLOW, true>)
                           : resident_slots(partial_kernel<D, G, PAGED, MODE_SLOW, false>);
    a.plan = plan_splits(a.max_len, a.batch_n * a.Hkv, slots, a.plan.stride, 1 << 30);
  }
  PartialArgs p{};
  p.B = a.B; p.max_len = a.max_len;
  p.kv = a.kv; p.seq_len = a.seq_len; p.batch_ids = a.batch_ids; p.q = a.q; p.Hq = a.Hq;
  p.chunk = a.plan.chunk; p.stride = a.plan.stride; p.part_o = a.part_o; p.part_ml = a.part_ml;
  p.logits = a.logits; p.lld = a.lld; p.key_norm = a.key_norm; p.ld = a.ld;
  p.qscale = kLog2e / sqrtf((float)D);
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
hipError_t fast_t(const AttnLaunch &a_in, hipStream_t st) {
  AttnLaunch a = a_in;
  {
    const long long L = (long long)std::min(a.n_sink, a.max_len) + std::min(a.window, a.max_len) + a.sel_k;
    const int slots = resident_slots(partial_kernel<D, G, PAGED, MODE_FAST, false>);
    a.plan = plan_splits(L, a.batch_n * a.Hkv, slots, a.plan.stride, kMaxFastChunk);
  }
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

SplitPlan plan_splits(long long L, int pairs, int slots, int stride, int max_chunk) {
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

hipError_t launch_slow(const AttnLaunch &a, hipStream_t st) { SFI_DISPATCH(slow_t, a, st); }
hipError_t launch_fast(const AttnLaunch &a, hipStream_t st) {
  SFI_DISPATCH(fast_t, a, st);
}

}  // namespace sfi
