// Device helpers shared by the libsfi kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfi {

constexpr float kLog2e = 1.4426950408889634f;
// Finite "minus infinity" for running maxima: exp2(kNegBig - x) == 0 for any
// finite logit x, and kNegBig - kNegBig == 0 keeps empty states NaN-free.
constexpr float kNegBig = -1.0e30f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// a.lo*b.lo + a.hi*b.hi + c: the bf16 products are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR (8 or 16) lanes; every lane of the group
// receives the group's sum.  DPP row permutes only, so no LDS traffic.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16, "group of 8 or 16 lanes");
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror: the other quad of each 8
  if constexpr (LPR == 16) x += dpp_f32<0x140>(x);  // row_mirror: other 8 of 16
  return x;
}

// Lane exchange across lane ^ OFF (OFF = 16 or 32) by the gfx950 permlane
// swaps, which move data between lane halves in the VALU instead of through
// the LDS crossbar.  permlaneOFF_swap(a, b) swaps a of the upper lanes with b
// of the lower lanes, so afterwards a lower lane holds (own a, partner's a)
// and an upper lane (partner's b, own b): the sum of the two results is, in
// every lane, that lane's kept value (a below, b above) plus the partner's
// copy of it -- one step of a reduce-scatter, with no per-lane select.
template <int OFF>
__device__ __forceinline__ float xsum_scatter(float a, float b) {
  static_assert(OFF == 16 || OFF == 32, "lane halves of a row pair or of the wave");
  uint32_t r0, r1;
  if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    r0 = r[0];
    r1 = r[1];
  }
  return __uint_as_float(r0) + __uint_as_float(r1);
}

// x[lane] + x[lane ^ OFF] and max(x[lane], x[lane ^ OFF]) in every lane.
template <int OFF>
__device__ __forceinline__ float xsum(float x) { return xsum_scatter<OFF>(x, x); }

template <int OFF>
__device__ __forceinline__ float xmax(float x) {
  static_assert(OFF == 16 || OFF == 32, "lane halves of a row pair or of the wave");
  uint32_t r0, r1;
  if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    r0 = r[0];
    r1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    r0 = r[0];
    r1 = r[1];
  }
  return fmaxf(__uint_as_float(r0), __uint_as_float(r1));
}

// Location of one cached K/V row.
struct KVView {
  const uint16_t *k;
  const uint16_t *v;
  const int32_t *page_table;  // nullptr: contiguous [B][Hkv][cap][D]
  int32_t page_shift;         // log2(page_size)
  int32_t max_pages;
  int32_t num_pages;
  int32_t Hkv;
  int32_t cap;
  // The step's own new row per (sequence, kv head), [B][Hkv][D], or null.
  // Set, a decode kernel takes row seq_len - 1 from here and the workgroup
  // that owns that row's list position stores it into the cache.
  const uint16_t *k_new;
  const uint16_t *v_new;
  // Key-norm statistics [B][Hkv][2] (sum and sum of squares of the norms of
  // the cached rows, fp64), or null.
  double *nstat;
};

template <int D, bool PAGED>
__device__ __forceinline__ size_t kv_row(const KVView &kv, int b, int g, int j) {
  if constexpr (!PAGED) {
    return ((size_t)(b * kv.Hkv + g) * (size_t)kv.cap + (size_t)j) * D;
  } else {
    int pg = kv.page_table[(size_t)b * kv.max_pages + (j >> kv.page_shift)];
    pg = min(max(pg, 0), kv.num_pages - 1);
    const int off = j & ((1 << kv.page_shift) - 1);
    return ((((size_t)pg * kv.Hkv + g) << kv.page_shift) + (size_t)off) * D;
  }
}

// Sequence id of batch entry i (nullptr list: identity); -1 when out of range.
__device__ __forceinline__ int batch_seq(const int32_t *ids, int i, int B) {
  const int b = ids ? ids[i] : i;
  return (b >= 0 && b < B) ? b : -1;
}

// Blocks of a grid share over (head, batch entry) pairs: P = H x Z pairs,
// S blocks per pair, w the block's index in the share.  Workgroups go to
// the 8 XCDs round-robin by linear id, so with xcd set, a share starting at
// a linear id that is a multiple of 8 and P a multiple of 8, block w takes
// pair (w % 8) + 8 ((w / 8) / S) and block (w / 8) % S: every block of a
// pair runs on XCD pair % 8, where a later kernel's blocks of the same pair
// also run and find what this one wrote in that XCD's L2.  Otherwise pair
// w / S, block w % S.  The fast steps' gathers, the finalize blocks and the
// selector gain from it; the long contiguous streams of dense and slow
// steps measured slower with it (a 128K dense step 331 -> 346 us), so their
// partial blocks keep the plain order.
#ifndef SFI_XCD_MAP
#define SFI_XCD_MAP 1
#endif
struct PairBlock {
  int blk, h, z;
};
__device__ __forceinline__ PairBlock pair_block(int w, int S, int H, int Z, bool xcd = true) {
  int pair;
  int blk;
  if (SFI_XCD_MAP && xcd && ((H * Z) & 7) == 0) {
    const int k = w >> 3;
    const int q = k / S;
    pair = (w & 7) + 8 * q;
    blk = k - q * S;
  } else {
    pair = w / S;
    blk = w - pair * S;
  }
  return {blk, pair % H, pair / H};
}

// Split counts of a grid share planned from the lengths of its listed
// entries (host-known): entry z of the batch list takes splits [0, c_z) of
// every kv head, cum[z] = c_0 + ... + c_{z-1}.  The share's blocks are
// numbered w = (cum[z] + s) * Hkv + g (heads fastest), so no block lands
// past an entry's rows.  n = 0: no table (every entry takes the planned
// number of splits and the blocks past its rows exit at once).
constexpr int kMaxListed = 256;
struct WorkTable {
  int n;
  uint16_t cum[kMaxListed + 1];
};

// Entry, head and split of block w of a tabled share.  The entry is the
// number of z in [1, n) with cum[z] <= e: each lane tests up to 4 entries
// and ballots count them, so the table's loads are in flight together and
// the entry's own prefix sum comes from a lane (a binary search made each
// block wait on ~log2(n) dependent loads of the kernel arguments).
__device__ __forceinline__ PairBlock table_block(const WorkTable &t, int w, int Hkv) {
  const int e = w / Hkv;
  const int lane = (int)(threadIdx.x & 63);
  int c[kMaxListed / 64];
#pragma unroll
  for (int i = 0; i < kMaxListed / 64; ++i) {
    const int zi = 1 + lane + 64 * i;
    c[i] = (zi < t.n) ? (int)t.cum[zi] : 0x7fffffff;
  }
  int z = 0;
#pragma unroll
  for (int i = 0; i < kMaxListed / 64; ++i) z += __popcll(__ballot(c[i] <= e));
  // cum[z] is entry z's value among the lanes' (z >= 1), cum[0] = 0
  int base = 0;
  if (z > 0) {
    const int zi = z - 1;
    int v = c[0];
#pragma unroll
    for (int i = 1; i < kMaxListed / 64; ++i) v = ((zi >> 6) == i) ? c[i] : v;
    base = __builtin_amdgcn_readlane(v, zi & 63);
  }
  return {e - base, w - e * Hkv, z};
}

// Splits of entry z: its table count, or the planned number.
__device__ __forceinline__ int entry_splits(const WorkTable &t, int z, int planned) {
  return t.n > 0 ? (int)t.cum[z + 1] - (int)t.cum[z] : planned;
}

// Linear id of the block in its grid (x fastest, the dispatch order).
__device__ __forceinline__ int linear_block() {
  return (int)(blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z));
}

// Cached length of sequence b clamped to [0, max_len].
__device__ __forceinline__ int clamp_len(const int32_t *seq_len, int b, int max_len) {
  return min(max(seq_len[b], 0), max_len);
}

// Order-preserving map float -> uint32 (larger float -> larger key).
// 2^x by the hardware instruction (v_exp_f32).  It matches the library's
// exp2f wherever the result is a normal number; below 2^-126 it returns 0
// instead of a denormal.  Every use either adds the result to a sum that
// holds a term of at least 1 or weights a term that is then negligible.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Prior weight of key j: exp(-norm_coef z_j) (1 + exp(-(t - j)/tau)) with
// z_j = (nu_j - mu)/sd, as powers of two (cz = -norm_coef log2(e)/sd,
// ct = log2(e)/tau, tq = t).  Every kernel that forms the weights or their
// sum calls this one function, so sums and keys agree bit for bit.
__device__ __forceinline__ float prior_w(float nu, int j, float muf, float cz, float tq, float ct) {
  return exp2_hw(cz * (nu - muf)) * (1.0f + exp2_hw(((float)j - tq) * ct));
}

// Row constants of the prior from fp64 sums of the key norms over n keys:
// muf = mean, cz = -norm_coef log2(e) / population std (0 when the std is 0).
__device__ __forceinline__ void prior_consts(double s1, double s2, int n, float norm_coef, float *muf,
                                             float *cz) {
  const double mu = s1 / n;
  const double var = fmax(s2 / n - mu * mu, 0.0);
  const double sd = sqrt(var);
  *muf = (float)mu;
  const float isd = sd > 0.0 ? (float)(1.0 / sd) : 0.0f;
  *cz = -norm_coef * isd * kLog2e;
}

__device__ __forceinline__ uint4 ldg16(const uint16_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// Sum of squares of 8 bf16 values (one 16-byte slice of a row).
__device__ __forceinline__ float slice_sumsq(uint4 t) {
  float ss = dot2_bf16(t.x, t.x, 0.f);
  ss = dot2_bf16(t.y, t.y, ss);
  ss = dot2_bf16(t.z, t.z, ss);
  return dot2_bf16(t.w, t.w, ss);
}

// Euclidean norm of a row of D bf16 values from its 16-byte slices held by
// lanes 0 .. D/8 - 1 of the wave (t; other lanes pass anything): a sum over
// the wave, so every lane returns it.  The one formula the key-norm
// statistics use for a row they add.
template <int D>
__device__ __forceinline__ float wave_row_norm(uint4 t) {
  float ss = ((threadIdx.x & 63) < D / 8) ? slice_sumsq(t) : 0.f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  return __builtin_amdgcn_sqrtf(ss);
}

// 16-byte load marked non-temporal: for rows streamed once per call (dense
// and slow steps), so they do not displace reused data in the caches.
__device__ __forceinline__ uint4 ldg16_stream(const uint16_t *p) {
  typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
  const u32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

}  // namespace sfi
