// Multi-query verification attention with aggregated logits on gfx950 MFMA.
//
// Vegas (gist.science/it/paper/2602.07223), section 2: the verification pass
// runs full attention for the gamma+1 verified tokens and its logits pick the
// keys the next draft phase attends; section 2.A: the selection score of a
// prefix key is its pre-softmax logit summed over the verified queries and
// all query heads; section 2.B: Collect-2-Query sums only the first draft
// query and the bonus query.  Logits are q.k/sqrt(d) (section 3: taken before
// the softmax).
//
// One kv head serves R = (Hq/Hkv) * T query rows (32 for GQA 4:1 and T = 8),
// so a 32-key tile is a dense 32 x 32 x d contraction: it runs on
// v_mfma_f32_32x32x16_bf16 with keys on the M axis (S^T = K Q^T).  In that
// orientation
//   * the K tile is the A operand and is loaded straight from HBM into
//     registers (lane: one key, 8 consecutive dims per k-step);
//   * the accumulator gives every lane one query column and 16 keys, so the
//     per-row softmax max/sum needs a single cross-half exchange;
//   * the same accumulator, re-typed to bf16, is already the B operand of
//     O^T = V^T P^T (P is split into a bf16 high part and a bf16 residual, so
//     P V keeps ~16 mantissa bits);
//   * V^T's A operand is gathered as 32-bit (even, odd dim) pairs, one dword
//     per key per lane, and repacked into the even-dim and odd-dim m-tiles;
//   * the aggregate is a masked sum of accumulator columns, done as a
//     16-shuffle reduce-scatter inside each 32-lane half.
// Each wave owns a contiguous key range and writes its own (m, Z, O) partial;
// a finalize kernel merges them in a fixed order and sums the per-kv-head
// aggregates over kv heads.
#include <algorithm>

#include "sfi_internal.hpp"

namespace sfi {
namespace {


typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kVThreads = 256;
constexpr int kVWaves = kVThreads / 64;

struct VArgs {
  KVView kv;
  int B, max_len;
  const int32_t *seq_len;
  const int32_t *batch_ids;
  const uint16_t *q;  // [B][T][Hq][D]
  int Hq, T;
  uint32_t row_mask;
  int wchunk;         // keys per wave
  int stride;         // wave partials per row
  float *part_o;      // [B][T*Hq][stride][D]
  float *part_ml;     // [B][T*Hq][stride][2]
  float *part_agg;    // [B][Hkv][lld]
  int lld;
  float qscale;       // log2(e)/sqrt(d)
  float lscale;       // 1/sqrt(d)
  // raw-logit emission: pre-softmax logits of the collected rows,
  // [B][nraw][Hq][raw_ld] (row index = rank of the row among row_mask's bits)
  float *raw;
  int raw_ld, nraw;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  u32x4_t v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Key (within a 32-key tile) held by accumulator element r of a lane in half hs.
__device__ __forceinline__ int acc_key(int r, int hs) { return 8 * (r >> 2) + 4 * hs + (r & 3); }

template <int D, int G, bool PAGED, bool RAW = false>
__global__ __launch_bounds__(kVThreads) void verify_partial_kernel(VArgs a) {
  constexpr int KK = D / 16;  // k-steps of Q K^T
  constexpr int MT = D / 32;  // m-tiles of O^T
  constexpr int NP = MT / 2;  // (even, odd) m-tile pairs

  const int b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (b < 0) return;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hs = lane >> 5;
  const int n = clamp_len(a.seq_len, b, a.max_len);
  const int T = a.T;
  const int R = G * T;
  // The workgroup owns keys [K0, k1), kVWaves * wchunk of them, and wave w
  // takes its 32-key tiles w, w + kVWaves, ...: the workgroup sweeps one
  // contiguous range of K and of V (one stream per workgroup, not per wave,
  // measured faster), while each wave keeps its own (m, Z, O) partial.
  const int widx = blockIdx.x * kVWaves + wave;
  const int K0 = blockIdx.x * kVWaves * a.wchunk;
  if (K0 >= n) return;
  const int k1 = min(n, K0 + kVWaves * a.wchunk);
  const int k0 = K0 + 32 * wave;  // this wave's first tile

  // Query column of this lane: verify row jt, head jh of the group.
  const bool colv = col < R;
  const int jt = colv ? col / G : 0;
  const int jh = colv ? col % G : 0;
  const int lim = n - T + jt;  // last visible key of row jt
  const float amask = (colv && ((a.row_mask >> jt) & 1u)) ? 1.f : 0.f;
  const int prefix = n - T;    // aggregate covers keys < prefix
  // raw-logit emission: this lane's column writes its logits when its row is
  // collected, at row rank(jt) of the collected rows
  float *rawp = nullptr;
  if constexpr (RAW) {
    if (amask != 0.f) {
      const int rr = __popc(a.row_mask & ((1u << jt) - 1u));
      rawp = a.raw + (((size_t)b * a.nraw + rr) * a.Hq + g * G + jh) * a.raw_ld;
    }
  }

  bf16x8_t qb[KK];
  {
    const uint16_t *qp = a.q + (((size_t)b * T + jt) * a.Hq + g * G + jh) * D + 8 * hs;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 t = colv ? ldg16(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qb[kk] = as_bf16x8(t);
    }
  }

  f32x16_t o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mt][r] = 0.f;
  float m = kNegBig, z = 0.f;
  const size_t aggrow = ((size_t)b * a.kv.Hkv + g) * a.lld;

  // One 32-key tile: the K rows as the A operand of S^T = K Q^T, and the
  // (even, odd)-dim dwords of the V rows this lane needs for O^T's A operand.
  // K and V arrive as whole 128-byte lines (8 lanes per line, 16 bytes
  // each, the lines of 8 keys per instruction: D/16 instructions per tile
  // and operand) and are rearranged through the wave's LDS slice: K into
  // the MFMA layout of S^T (lane: one key, 8 consecutive dims per k-step),
  // V into the (even, odd)-dim dwords O^T's A operand needs.  With every
  // load covering whole lines they are loaded non-temporally, and a tile
  // takes 16 load instructions instead of 40 (V read straight from HBM as
  // dwords took 32).  16 sequences x 64K: 852 -> ~760 us with K through LDS;
  // a K load straight in the MFMA layout reads 32 bytes of 32 lines per
  // instruction, and the non-temporal hint made that 30 % slower.
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  struct Tile {
    uint4 kraw[KK];
    uint4 vraw[KK];
  };
  __shared__ uint4 s_kt[kVWaves][32 * CPR];
  __shared__ uint4 s_vt[kVWaves][32 * CPR];
  uint4 *kt = s_kt[wave];
  uint4 *vt = s_vt[wave];
  const uint32_t *vt32 = reinterpret_cast<const uint32_t *>(vt);
  // Every lane issues its loads unconditionally: a key past the range reads
  // row k1 - 1 instead (k1 > K0, so it exists) and is masked in
  // consume().  Loads behind per-lane branches would leave the number of
  // loads in flight unknown at compile time and every later wait would have
  // to drain them all, which would collapse the two-stage pipeline below.
  auto load_tile = [&](Tile &t, int kb) {
#pragma unroll
    for (int i = 0; i < KK; ++i) {
      const int L = i * 8 + (lane >> 3);  // line of the tile: key L % 32, line L / 32 of its row
      const int key = min(kb + (L & 31), k1 - 1);
      const int ch = (L >> 5) * 8 + (lane & 7);
      const size_t row = kv_row<D, PAGED>(a.kv, b, g, key) + 8 * ch;
      t.kraw[i] = ldg16_stream(a.kv.k + row);
      t.vraw[i] = ldg16_stream(a.kv.v + row);
    }
  };
  // Lazy rescaling: the running reference m only moves when a logit exceeds
  // it by more than kSlack (log2 units), so p = 2^(l - m) stays <= 2^kSlack
  // and the accumulators are rescaled on few tiles.
  constexpr float kSlack = 8.0f;
  auto consume = [&](const Tile &t, int kb) {
    // K tile through LDS: row-major [32 keys][CPR chunks], chunk index
    // XOR-swizzled by the key (spreads a k-step's 32 rows over the banks);
    // only this wave touches its slice, and LDS operations of a wave run in
    // order, so the wave barriers (compiler ordering only) suffice.
    bf16x8_t ka[KK];
#pragma unroll
    for (int i = 0; i < KK; ++i) {
      const int L = i * 8 + (lane >> 3);
      const int key = L & 31, ch = (L >> 5) * 8 + (lane & 7);
      kt[key * CPR + (ch ^ (key & (CPR - 1)))] = t.kraw[i];
      vt[key * CPR + (ch ^ (key & (CPR - 1)))] = t.vraw[i];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int ch = 2 * kk + hs;
      ka[kk] = as_bf16x8(kt[col * CPR + (ch ^ (col & (CPR - 1)))]);
    }
    __builtin_amdgcn_wave_barrier();
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qb[kk], s, 0, 0, 0);

    // Raw-logit emission: the lane's 16 logits of its column, 4 runs of 4
    // consecutive keys (keys of the prefix only).
    if constexpr (RAW) {
      if (rawp) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int key = kb + acc_key(4 * r4, hs);
          const float4 v = make_float4(s[4 * r4] * a.lscale, s[4 * r4 + 1] * a.lscale, s[4 * r4 + 2] * a.lscale,
                                       s[4 * r4 + 3] * a.lscale);
          if (key + 3 < prefix && key + 3 < k1 && (a.raw_ld & 3) == 0) {
            *reinterpret_cast<float4 *>(rawp + key) = v;
          } else {
            if (key < prefix && key < k1) rawp[key] = v.x;
            if (key + 1 < prefix && key + 1 < k1) rawp[key + 1] = v.y;
            if (key + 2 < prefix && key + 2 < k1) rawp[key + 2] = v.z;
            if (key + 3 < prefix && key + 3 < k1) rawp[key + 3] = v.w;
          }
        }
      }
    }
    // Aggregate: masked column sum, reduce-scattered over the 32 lanes of the half.
    if (!RAW && a.part_agg) {
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = s[r] * amask;
      const bool b4 = (col & 16) != 0, b3 = (col & 8) != 0, b2 = (col & 4) != 0, b1 = (col & 2) != 0;
      float w8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float keep = b4 ? v[8 + i] : v[i];
        const float send = b4 ? v[i] : v[8 + i];
        w8[i] = keep + __shfl_xor(send, 16);
      }
      float w4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float keep = b3 ? w8[4 + i] : w8[i];
        const float send = b3 ? w8[i] : w8[4 + i];
        w4[i] = keep + __shfl_xor(send, 8);
      }
      float w2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float keep = b2 ? w4[2 + i] : w4[i];
        const float send = b2 ? w4[i] : w4[2 + i];
        w2[i] = keep + __shfl_xor(send, 4);
      }
      float w1 = (b1 ? w2[1] : w2[0]) + __shfl_xor(b1 ? w2[0] : w2[1], 2);
      w1 += __shfl_xor(w1, 1);
      const int r = 8 * (int)b4 + 4 * (int)b3 + 2 * (int)b2 + (int)b1;
      const int key = kb + acc_key(r, hs);
      if ((col & 1) == 0 && key < k1 && key < prefix) a.part_agg[aggrow + key] = w1 * a.lscale;
    }

    // Online softmax of column col over this tile (16 keys here, 16 in lane^32).
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + acc_key(r, hs);
      const bool ok = key < k1 && key <= lim;
      sv[r] = ok ? s[r] * a.qscale : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool need = mx > m + kSlack;
    if (__any(need)) {
      const float mn = need ? mx : m;
      const float sc = exp2_hw(m - mn);
      m = mn;
      z *= sc;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][r] *= sc;
    }

#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t phi, plo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2_hw(sv[8 * ks + e] - m);
        z += p;
        const float ph = __uint_as_float(__float_as_uint(p) & 0xffff0000u);
        phi[e] = (__bf16)ph;
        plo[e] = (__bf16)(p - ph);
      }
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        // the (even, odd)-dim dword of dims 2 col, 2 col + 1 (+ 64 pp) of
        // the 8 keys of k-step ks held by this lane's half, from the V tile
        uint32_t vw[8];
        const int dw = col + 32 * pp, chv = dw >> 2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = 16 * ks + acc_key(e, hs);
          vw[e] = vt32[(key * CPR + (chv ^ (key & (CPR - 1)))) * 4 + (dw & 3)];
        }
        u32x4_t ev, od;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t w0 = vw[2 * i], w1 = vw[2 * i + 1];
          ev[i] = (w0 & 0xffffu) | (w1 << 16);
          od[i] = (w0 >> 16) | (w1 & 0xffff0000u);
        }
        const bf16x8_t ae = __builtin_bit_cast(bf16x8_t, ev);
        const bf16x8_t ao = __builtin_bit_cast(bf16x8_t, od);
        o[2 * pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ae, phi, o[2 * pp], 0, 0, 0);
        o[2 * pp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ae, plo, o[2 * pp], 0, 0, 0);
        o[2 * pp + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, phi, o[2 * pp + 1], 0, 0, 0);
        o[2 * pp + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, plo, o[2 * pp + 1], 0, 0, 0);
      }
    }
  };

  // Two tiles in flight: the loads of one overlap the MFMA and softmax work
  // of the other.  Tiles past k1 are fully masked (p = 0, no aggregate write);
  // a wave with no tile at all leaves Z = 0, which the combine skips.
  constexpr int TS = 32 * kVWaves;  // key step between a wave's tiles
  if (k0 < k1) {
    Tile ta, tb;
    load_tile(ta, k0);
    for (int kb = k0; kb < k1; kb += 2 * TS) {
      load_tile(tb, kb + TS);
      consume(ta, kb);
      load_tile(ta, kb + 2 * TS);
      consume(tb, kb + TS);
    }
  }

  const float zt = z + __shfl_xor(z, 32);
  if (colv) {
    const size_t slot = ((size_t)b * T * a.Hq + (size_t)jt * a.Hq + g * G + jh) * a.stride + widx;
    float *op = a.part_o + slot * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) op[64 * (mt >> 1) + 2 * acc_key(r, hs) + (mt & 1)] = o[mt][r];
    if (hs == 0) {
      a.part_ml[slot * 2 + 0] = m;
      a.part_ml[slot * 2 + 1] = zt;
    }
  }
}

struct VFinal {
  int B, max_len;
  const int32_t *seq_len;
  const int32_t *batch_ids;
  int Hq, Hkv, T, wchunk, stride;
  const float *part_o;
  const float *part_ml;
  float *out;
  const float *part_agg;
  int lld;
  float *agg;
  int ld;
  float *rstat;  // [B][T*Hq][2] merged (reference, sum) per row, or null
};

// grid.x = T*Hq rows, one block of D threads each: fixed-order merge.
template <int D>
__global__ __launch_bounds__(D) void verify_combine_kernel(VFinal a) {
  const int b = batch_seq(a.batch_ids, blockIdx.y, a.B);
  if (b < 0) return;
  const int row = blockIdx.x;  // t*Hq + h
  const int n = clamp_len(a.seq_len, b, a.max_len);
  // every wave of the workgroups that cover [0, n); waves without keys hold Z = 0
  const int S = (n + kVWaves * a.wchunk - 1) / (kVWaves * a.wchunk) * kVWaves;
  const size_t base = ((size_t)b * a.T * a.Hq + row) * a.stride;
  float M = kNegBig;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[(base + s) * 2]);
  float Z = 0.f, o = 0.f;
  const int e = threadIdx.x;
  for (int s = 0; s < S; ++s) {
    const float zs = a.part_ml[(base + s) * 2 + 1];
    if (zs > 0.f) {
      const float w = exp2_hw(a.part_ml[(base + s) * 2] - M);
      Z = fmaf(zs, w, Z);
      o = fmaf(a.part_o[(base + s) * D + e], w, o);
    }
  }
  a.out[((size_t)b * a.T * a.Hq + row) * D + e] = (Z > 0.f) ? o / Z : 0.f;
  if (a.rstat && e == 0) {
    a.rstat[((size_t)b * a.T * a.Hq + row) * 2 + 0] = M;
    a.rstat[((size_t)b * a.T * a.Hq + row) * 2 + 1] = Z;
  }
}

// Raw-logit mode: agg[b][i] = sum over the collected rows and all query heads
// (fixed order) of the emitted logits, i < n - T.
__global__ __launch_bounds__(256) void verify_raw_agg_kernel(VFinal a, const float *raw, int raw_ld, int nraw) {
  const int b = batch_seq(a.batch_ids, blockIdx.y, a.B);
  if (b < 0) return;
  const int n = clamp_len(a.seq_len, b, a.max_len);
  const int P = n - a.T;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < P; i += gridDim.x * 256) {
    float s = 0.f;
    for (int r = 0; r < nraw * a.Hq; ++r) s += raw[((size_t)b * nraw * a.Hq + r) * raw_ld + i];
    a.agg[(size_t)b * a.ld + i] = s;
  }
}

// agg[b][i] = sum over kv heads (fixed order) of the per-head partials, i < n - T.
__global__ __launch_bounds__(256) void verify_agg_kernel(VFinal a) {
  const int b = batch_seq(a.batch_ids, blockIdx.y, a.B);
  if (b < 0) return;
  const int n = clamp_len(a.seq_len, b, a.max_len);
  const int P = n - a.T;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < P; i += gridDim.x * 256) {
    float s = 0.f;
    for (int g = 0; g < a.Hkv; ++g) s += a.part_agg[((size_t)b * a.Hkv + g) * a.lld + i];
    a.agg[(size_t)b * a.ld + i] = s;
  }
}

// Evidence over the verify rows used as a slow step's observation window:
// for every key j < n of kv head g,
//   f_j = (1 / (T G)) * sum over the rows t that see j and the heads h of the
//         group of 2^(l_thj - M_th) / Z_th,
// with (M_th, Z_th) the row's merged softmax reference and sum (log2 domain)
// from the combine kernel.  The keys are read again (K only) and S^T = K Q^T
// is recomputed tile by tile on MFMA as in verify_partial_kernel; the column
// sums use the aggregate's reduce-scatter.  Optionally writes the key norms.
template <int D, int G, bool PAGED>
__global__ __launch_bounds__(kVThreads) void window_evidence_kernel(VArgs a, const float *rstat,
                                                                    float *evidence, float *key_norm,
                                                                    int ld) {
  constexpr int KK = D / 16;
  const int b = batch_seq(a.batch_ids, blockIdx.z, a.B);
  if (b < 0) return;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hs = lane >> 5;
  const int n = clamp_len(a.seq_len, b, a.max_len);
  const int T = a.T;
  const int R = G * T;
  const int K0 = blockIdx.x * kVWaves * a.wchunk;
  if (K0 >= n) return;
  const int k1 = min(n, K0 + kVWaves * a.wchunk);
  const int k0 = K0 + 32 * wave;
  const bool colv = col < R;
  const int jt = colv ? col / G : 0;
  const int jh = colv ? col % G : 0;
  const int lim = n - T + jt;  // last key row jt sees
  float Mc = 0.f, wc = 0.f;
  if (colv) {
    const size_t rrow = ((size_t)b * T + jt) * a.Hq + g * G + jh;
    Mc = rstat[rrow * 2];
    const float Zc = rstat[rrow * 2 + 1];
    wc = (Zc > 0.f) ? 1.0f / (Zc * (float)R) : 0.f;
  }
  bf16x8_t qb[KK];
  {
    const uint16_t *qp = a.q + (((size_t)b * T + jt) * a.Hq + g * G + jh) * D + 8 * hs;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 t = colv ? ldg16(qp + 16 * kk) : make_uint4(0, 0, 0, 0);
      qb[kk] = as_bf16x8(t);
    }
  }
  const size_t erow = ((size_t)b * a.kv.Hkv + g) * ld;
  struct KTile {
    bf16x8_t ka[KK];
  };
  // loads issued unconditionally (a key past the range reads row k1 - 1)
  auto load_tile = [&](KTile &t, int kb) {
    const int key = min(kb + col, k1 - 1);
    const uint16_t *kp = a.kv.k + kv_row<D, PAGED>(a.kv, b, g, key) + 8 * hs;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) t.ka[kk] = as_bf16x8(ldg16(kp + 16 * kk));
  };
  auto consume = [&](const KTile &t, int kb) {
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t.ka[kk], qb[kk], s, 0, 0, 0);
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + acc_key(r, hs);
      const bool ok = key < k1 && key <= lim;
      v[r] = ok ? exp2_hw(s[r] * a.qscale - Mc) * wc : 0.f;
    }
    const bool b4 = (col & 16) != 0, b3 = (col & 8) != 0, b2 = (col & 4) != 0, b1 = (col & 2) != 0;
    float w8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float keep = b4 ? v[8 + i] : v[i];
      const float send = b4 ? v[i] : v[8 + i];
      w8[i] = keep + __shfl_xor(send, 16);
    }
    float w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float keep = b3 ? w8[4 + i] : w8[i];
      const float send = b3 ? w8[i] : w8[4 + i];
      w4[i] = keep + __shfl_xor(send, 8);
    }
    float w2[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float keep = b2 ? w4[2 + i] : w4[i];
      const float send = b2 ? w4[i] : w4[2 + i];
      w2[i] = keep + __shfl_xor(send, 4);
    }
    float w1 = (b1 ? w2[1] : w2[0]) + __shfl_xor(b1 ? w2[0] : w2[1], 2);
    w1 += __shfl_xor(w1, 1);
    const int r = 8 * (int)b4 + 4 * (int)b3 + 2 * (int)b2 + (int)b1;
    const int key = kb + acc_key(r, hs);
    if ((col & 1) == 0 && key < k1) evidence[erow + key] = w1;
    if (key_norm) {
      // lane (col, hs) holds half of key kb + col's dims
      float nn = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)t.ka[kk][e];
          nn = fmaf(x, x, nn);
        }
      nn += __shfl_xor(nn, 32);
      if (hs == 0 && kb + col < k1) key_norm[erow + kb + col] = sqrtf(nn);
    }
  };
  constexpr int TS = 32 * kVWaves;
  if (k0 < k1) {
    KTile ta, tb;
    load_tile(ta, k0);
    for (int kb = k0; kb < k1; kb += 2 * TS) {
      load_tile(tb, kb + TS);
      consume(ta, kb);
      load_tile(ta, kb + 2 * TS);
      consume(tb, kb + TS);
    }
  }
}

template <int D, int G, bool PAGED>
hipError_t verify_t(const VerifyLaunch &L, hipStream_t st) {
  VArgs a{};
  a.B = L.B; a.max_len = L.max_seq_len;
  a.kv = L.kv; a.seq_len = L.seq_len; a.batch_ids = L.batch_ids; a.q = L.q;
  a.Hq = L.Hq; a.T = L.T; a.row_mask = L.row_mask;
  a.wchunk = L.plan.chunk; a.stride = L.plan.stride;
  a.part_o = L.part_o; a.part_ml = L.part_ml; a.part_agg = L.part_agg; a.lld = L.lld;
  a.qscale = kLog2e / sqrtf((float)D);
  a.lscale = 1.0f / sqrtf((float)D);
  a.raw = L.raw; a.raw_ld = L.raw_ld; a.nraw = __builtin_popcount(L.row_mask);
  const int wgs = (L.plan.splits + kVWaves - 1) / kVWaves;
  if (L.raw)
    hipLaunchKernelGGL((verify_partial_kernel<D, G, PAGED, true>), dim3(wgs, L.Hkv, L.batch_n),
                       dim3(kVThreads), 0, st, a);
  else
    hipLaunchKernelGGL((verify_partial_kernel<D, G, PAGED>), dim3(wgs, L.Hkv, L.batch_n),
                       dim3(kVThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  VFinal f{};
  f.B = L.B; f.max_len = L.max_seq_len;
  f.seq_len = L.seq_len; f.batch_ids = L.batch_ids; f.Hq = L.Hq; f.Hkv = L.Hkv; f.T = L.T;
  f.wchunk = L.plan.chunk; f.stride = L.plan.stride; f.part_o = L.part_o; f.part_ml = L.part_ml;
  f.out = L.out; f.part_agg = L.part_agg; f.lld = L.lld; f.agg = L.agg; f.ld = L.ld;
  f.rstat = L.rstat;
  hipLaunchKernelGGL((verify_combine_kernel<D>), dim3(L.T * L.Hq, L.batch_n), dim3(D), 0, st, f);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (L.evidence) {  // observation-window slow step: evidence instead of the aggregate
    hipLaunchKernelGGL((window_evidence_kernel<D, G, PAGED>), dim3(wgs, L.Hkv, L.batch_n), dim3(kVThreads), 0,
                       st, a, L.rstat, L.evidence, L.key_norm, L.ld);
    return hipGetLastError();
  }
  const int aggb = min(1024, (L.max_seq_len + 255) / 256);
  if (L.raw)
    hipLaunchKernelGGL(verify_raw_agg_kernel, dim3(aggb > 0 ? aggb : 1, L.batch_n), dim3(256), 0, st, f, L.raw,
                       L.raw_ld, a.nraw);
  else
    hipLaunchKernelGGL(verify_agg_kernel, dim3(aggb > 0 ? aggb : 1, L.batch_n), dim3(256), 0, st, f);
  return hipGetLastError();
}

}  // namespace

int verify_stride_for(int max_seq_len, int chunk) {
  // partial slots per row: every wave of the workgroups covering max_seq_len
  const int per_wg = kVWaves * chunk;
  return (max_seq_len + per_wg - 1) / per_wg * kVWaves;
}

namespace {

// Resident workgroups of the verify kernel on this device (cached per
// device and shape; the contiguous-cache kernel's, so paged caches get the
// same plan and bits).
template <int D, int G>
int verify_slots_t() {
  static int slots[16] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (slots[dev] == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, verify_partial_kernel<D, G, false>, kVThreads, 0) !=
            hipSuccess || nb < 1)
      nb = 1;
    slots[dev] = nb * device_cu_count();
  }
  return slots[dev];
}

int verify_slots(int d, int G) {
  switch (d * 16 + G) {
    case 64 * 16 + 1: return verify_slots_t<64, 1>();
    case 64 * 16 + 2: return verify_slots_t<64, 2>();
    case 64 * 16 + 4: return verify_slots_t<64, 4>();
    case 64 * 16 + 8: return verify_slots_t<64, 8>();
    case 128 * 16 + 1: return verify_slots_t<128, 1>();
    case 128 * 16 + 2: return verify_slots_t<128, 2>();
    case 128 * 16 + 4: return verify_slots_t<128, 4>();
    case 128 * 16 + 8: return verify_slots_t<128, 8>();
    default: return 256;
  }
}

}  // namespace

int verify_chunk_for(int B, int Hkv, int max_seq_len, int d, int G) {
  // Keys per wave.  The workgroups of all (sequence, kv head) pairs should
  // fill the resident slots in whole rounds: a plan that leaves a short last
  // round (say 2.25 rounds) runs its tail on a fraction of the chip.  So a
  // pair gets slots / pairs workgroups (at least one), and the chunk spreads
  // max_seq_len over them -- but a wave streams at least kMinChunk keys, so
  // its (m, Z, O) partial (R x (d+2) floats) stays a few percent of the K/V
  // bytes it reads.
  constexpr int kMinChunk = 512;
  const long long pairs = std::max(1LL, (long long)B * Hkv);
  const long long slots = verify_slots(d, G);
  const long long per_pair = std::max(1LL, slots / pairs);
  const long long keys_per_wg = (max_seq_len + per_pair - 1) / per_pair;
  long long chunk = (keys_per_wg + kVWaves - 1) / kVWaves;
  chunk = (chunk + 31) / 32 * 32;
  const long long small = ((long long)max_seq_len + kVWaves * 32 - 1) / (kVWaves * 32) * 32;  // one workgroup
  chunk = std::max(chunk, std::min<long long>(kMinChunk, small));
  return (int)std::max(32LL, chunk);
}

hipError_t launch_verify(const VerifyLaunch &L, hipStream_t st) {
  const bool pg = L.paged;
  switch (L.d * 16 + L.G) {
    case 64 * 16 + 1: return pg ? verify_t<64, 1, true>(L, st) : verify_t<64, 1, false>(L, st);
    case 64 * 16 + 2: return pg ? verify_t<64, 2, true>(L, st) : verify_t<64, 2, false>(L, st);
    case 64 * 16 + 4: return pg ? verify_t<64, 4, true>(L, st) : verify_t<64, 4, false>(L, st);
    case 64 * 16 + 8: return pg ? verify_t<64, 8, true>(L, st) : verify_t<64, 8, false>(L, st);
    case 128 * 16 + 1: return pg ? verify_t<128, 1, true>(L, st) : verify_t<128, 1, false>(L, st);
    case 128 * 16 + 2: return pg ? verify_t<128, 2, true>(L, st) : verify_t<128, 2, false>(L, st);
    case 128 * 16 + 4: return pg ? verify_t<128, 4, true>(L, st) : verify_t<128, 4, false>(L, st);
    case 128 * 16 + 8: return pg ? verify_t<128, 8, true>(L, st) : verify_t<128, 8, false>(L, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sfi
