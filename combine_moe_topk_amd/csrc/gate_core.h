// Device code of the top-K gate, shared by the gate kernel and the kernel
// that runs the gate and the layout's per-tile counts in one launch.  Not
// part of the ABI.
//
// "Efficient and portable mixture-of-experts communication", section
// "Introdución": the router yields a distribution over experts, the top-K
// scoring experts are kept, and their outputs are averaged with weights taken
// from that distribution.  Selection is by logit (softmax is monotone, so the
// chosen set is the same, and comparing the fp32 logits themselves cannot
// create ties that rounding of exp() would); equal logits go to the lower
// expert index; -0.0 ranks equal to +0.0.
//
// Layout: a group of G lanes (16, 32 or 64) owns one token.  Lane `sub` of
// the group holds the logits of experts sub, sub+G, sub+2G, ...  The path:
//
//  1. Threshold.  theta is a value that at least K of the token's logits
//     reach, so the K best are all at or above it: in each 16-lane row, the
//     ceil(K / rows)-th largest of the lanes' maxima (ranked with DPP
//     rotations), then the minimum over the group's rows.
//  2. Compaction.  The logits at or above theta (the candidates, typically
//     K to 2K of them) are written to LDS as 64-bit keys, (order-preserving
//     bits of the logit) << 32 | ~expert, so that a larger key means a larger
//     logit, then a lower index.  Each lane's slice of the list comes from a
//     DPP scan of the lanes' candidate counts.
//  3. Rank.  Lane i takes entry i (and entry i + G when there are more than
//     G candidates) and counts the entries with a larger key: that is its
//     rank, and ranks below K are the output, in rank order.
//
// A wave whose groups hold more than 2G candidates (many equal logits), or
// a theta of -inf, takes the general path instead: each lane keeps a sorted
// cache of its best candidates and K rounds of DPP group maxima pick the
// winners one at a time.  Both give the same result; the tests cover each.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace gate {


__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_bits(uint32_t o) {
  const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror.  Together they reduce a 16-lane row into every lane.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF,
                                               false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Combine the four 16-lane rows' results for groups of G = 32 or 64 lanes.
template <int G, bool MAX>
__device__ __forceinline__ uint32_t across_rows(uint32_t v) {
  if constexpr (G == 16) {
    return v;
  } else {
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0);
    const uint32_t r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32);
    const uint32_t r3 = __builtin_amdgcn_readlane(v, 48);
    const uint32_t a = MAX ? (r0 > r1 ? r0 : r1) : (r0 < r1 ? r0 : r1);
    const uint32_t b = MAX ? (r2 > r3 ? r2 : r3) : (r2 < r3 ? r2 : r3);
    if constexpr (G == 32) {
      return (threadIdx.x & 32) ? b : a;
    } else {
      return MAX ? (a > b ? a : b) : (a < b ? a : b);
    }
  }
}

// Same for floats, by comparison (no NaN reaches these).
template <int G, bool MAX>
__device__ __forceinline__ float across_rows_f(float v) {
  if constexpr (G == 16) {
    return v;
  } else {
    const int iv = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(iv, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(iv, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(iv, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(iv, 48));
    const float a = MAX ? (r1 > r0 ? r1 : r0) : (r1 < r0 ? r1 : r0);
    const float b = MAX ? (r3 > r2 ? r3 : r2) : (r3 < r2 ? r3 : r2);
    if constexpr (G == 32) {
      return (threadIdx.x & 32) ? b : a;
    } else {
      return MAX ? (b > a ? b : a) : (b < a ? b : a);
    }
  }
}

template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  v = max(v, dpp<kDppMirror>(v));
  return across_rows<G, true>(v);
}

template <int G>
__device__ __forceinline__ uint32_t group_min(uint32_t v) {
  v = min(v, dpp<kDppQuadXor1>(v));
  v = min(v, dpp<kDppQuadXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  v = min(v, dpp<kDppMirror>(v));
  return across_rows<G, false>(v);
}

// Row (16-lane) maximum or minimum of floats, in every lane of the row.
template <bool MAX>
__device__ __forceinline__ float row_reduce_f(float c) {
  c = MAX ? fmaxf(c, dppf<kDppQuadXor1>(c)) : fminf(c, dppf<kDppQuadXor1>(c));
  c = MAX ? fmaxf(c, dppf<kDppQuadXor2>(c)) : fminf(c, dppf<kDppQuadXor2>(c));
  c = MAX ? fmaxf(c, dppf<kDppHalfMirror>(c))
          : fminf(c, dppf<kDppHalfMirror>(c));
  c = MAX ? fmaxf(c, dppf<kDppMirror>(c)) : fminf(c, dppf<kDppMirror>(c));
  return c;
}

template <int G>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
  return v;
}

template <int R>
__device__ __forceinline__ float row_ror_f(float v) {
  return dppf<0x120 + R>(v);
}

// The kk-th largest of the 16 values of a DPP row (as a multiset), in every
// lane of the row.  A lane whose value has fewer than kk strictly larger
// values in the row holds a value >= the kk-th largest, and the kk-th
// largest itself is such a value, so it is the smallest of them.  The
// larger values are counted one row_ror rotation at a time.
__device__ __forceinline__ float row_kth_largest(float v, int kk) {
  int gt = 0;
#define MOE_RANK_STEP(R) gt += row_ror_f<R>(v) > v ? 1 : 0;
  MOE_RANK_STEP(1) MOE_RANK_STEP(2) MOE_RANK_STEP(3) MOE_RANK_STEP(4)
  MOE_RANK_STEP(5) MOE_RANK_STEP(6) MOE_RANK_STEP(7) MOE_RANK_STEP(8)
  MOE_RANK_STEP(9) MOE_RANK_STEP(10) MOE_RANK_STEP(11) MOE_RANK_STEP(12)
  MOE_RANK_STEP(13) MOE_RANK_STEP(14) MOE_RANK_STEP(15)
#undef MOE_RANK_STEP
  return row_reduce_f<false>(gt < kk ? v : __builtin_huge_valf());
}

// Inclusive sum over the lanes of a group (DPP: row_shr inside 16-lane rows,
// then row_bcast:15 and row_bcast:31 across rows).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
template <int G>
__device__ __forceinline__ int group_inclusive_scan(int v) {
  v = dpp_add<0x111, 0xF>(v);
  v = dpp_add<0x112, 0xF>(v);
  v = dpp_add<0x114, 0xF>(v);
  v = dpp_add<0x118, 0xF>(v);
  if constexpr (G >= 32) v = dpp_add<0x142, 0xA>(v);  // into rows 1 and 3
  if constexpr (G == 64) v = dpp_add<0x143, 0xC>(v);  // into rows 2 and 3
  return v;
}

// Orders the LDS accesses of one wave (its lanes exchange data through
// LDS; no other wave touches that region).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Candidate key: larger means larger logit, then lower expert index; 0 is
// below every real key (the smallest, -inf, has high word 0x007FFFFF).
__device__ __forceinline__ uint64_t cand_key(float v, int e) {
  return ((uint64_t)order_bits(v) << 32) | (uint32_t)~e;
}

constexpr int kCache = 4;  // D: cached (key, position) pairs per lane

// Sorted cache of a lane's best keys (key descending, position ascending),
// for the general path.
struct Cache {
  uint32_t key[kCache];
  int pos[kCache];
  int n;          // valid entries
  bool more;      // keys after the cache may remain
  uint32_t lk;    // last key given out (refills start strictly after it)
  int lp;         //   and its position

  // Insert (k, j); j comes in ascending order, so an equal key stays behind.
  // Branch-free: c[i] = k beats entry i (monotone in i, the cache being
  // sorted); entry i becomes entry i-1 where c[i-1], k where c[i] alone,
  // and stays otherwise.
  __device__ __forceinline__ void insert(uint32_t k, int j) {
    bool c[kCache];
#pragma unroll
    for (int i = 0; i < kCache; ++i) c[i] = k > key[i];
#pragma unroll
    for (int i = kCache - 1; i > 0; --i) {
      key[i] = c[i - 1] ? key[i - 1] : (c[i] ? k : key[i]);
      pos[i] = c[i - 1] ? pos[i - 1] : (c[i] ? j : pos[i]);
    }
    key[0] = c[0] ? k : key[0];
    pos[0] = c[0] ? j : pos[0];
  }

  // The D best candidate pairs among those after (lk, lp); with first, all
  // of them.  cand: bit j set when key j is a candidate.  A key position
  // where no lane of the wave has a candidate is skipped as a whole (a
  // wave-uniform branch).
  template <int C>
  __device__ __forceinline__ void fill(const uint32_t *keys, uint64_t cand,
                                       bool first) {
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
      key[i] = 0u;
      pos[i] = 0;
    }
    int found = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const bool mine = (cand >> j) & 1;
      if (!__any(mine)) continue;
      const uint32_t k = keys[j];
      const bool after = first || k < lk || (k == lk && j > lp);
      if (mine && after) {
        insert(k, j);
        ++found;
      }
    }
    n = found < kCache ? found : kCache;
    more = found > kCache;
  }

  __device__ __forceinline__ void pop() {
    lk = key[0];
    lp = pos[0];
#pragma unroll
    for (int i = 0; i < kCache - 1; ++i) {
      key[i] = key[i + 1];
      pos[i] = pos[i + 1];
    }
    key[kCache - 1] = 0u;
    --n;
  }
};

// The per-lane outcome: up to two selected experts, each with its output
// position (rank), expert index and weight.
struct Picks {
  int r0, e0, r1, e1;
  float l0, l1;  // logits
  float w0, w1;  // weights
  bool on0, on1;
};

// Rank the compacted candidates of the lane's group.  Lane sub takes entry
// sub (TWO: and entry sub + G); n entries are compared, n a multiple of 4
// and the same for the whole wave.  Empty entries hold 0, which every
// candidate beats, so an empty entry's rank is at least M >= K.
template <int G, bool TWO>
__device__ __forceinline__ void rank_entries(const uint64_t *ent, int sub,
                                             int n, int K, Picks &p) {
  const uint64_t a = ent[sub];
  const uint64_t b = TWO ? ent[sub + G] : 0ull;
  int ra = 0, rb = 0;
  for (int i = 0; i < n; i += 4) {
    const ulonglong2 x = *reinterpret_cast<const ulonglong2 *>(ent + i);
    const ulonglong2 y = *reinterpret_cast<const ulonglong2 *>(ent + i + 2);
    ra += (x.x > a) + (x.y > a) + (y.x > a) + (y.y > a);
    if constexpr (TWO) rb += (x.x > b) + (x.y > b) + (y.x > b) + (y.y > b);
  }
  p.on0 = ra < K;
  p.r0 = ra;
  p.e0 = (int)~(uint32_t)a;
  p.l0 = from_order_bits((uint32_t)(a >> 32));
  p.on1 = TWO && rb < K;
  p.r1 = rb;
  p.e1 = (int)~(uint32_t)b;
  p.l1 = from_order_bits((uint32_t)(b >> 32));
}

// LDS entries one wave needs for its groups' candidate lists.
template <int G>
constexpr int lds_entries_per_wave() {
  return (64 / G) * (2 * G + 2);
}

// Issue the loads of the lane's C logits of `row` (expert sub + j*G),
// clamped to the row unless FULL (E == G*C).  The values are not waited
// for; call pin() once they are needed.
template <int G, int C, bool FULL>
__device__ __forceinline__ void load_keys(const float *row, int sub, int E,
                                          float (&v)[C]) {
  if constexpr (FULL) {
    const float *base = row + sub;
#pragma unroll
    for (int j = 0; j < C; ++j) v[j] = base[j * G];
  } else {
#pragma unroll
    for (int j = 0; j < C; ++j) v[j] = row[min(sub + j * G, E - 1)];
  }
}

// The empty asm takes every loaded value as an operand, so the compiler
// cannot move a load into the branch of a later select (where it would
// wait for each load in turn: C memory round trips instead of one).
// Padding keys (expert >= E) become -inf.
template <int G, int C, bool FULL>
__device__ __forceinline__ void pin_keys(int sub, int E, float (&v)[C]) {
#pragma unroll
  for (int j = 0; j < C; ++j) asm volatile("" : "+v"(v[j]));
  if constexpr (!FULL) {
#pragma unroll
    for (int j = 0; j < C; ++j)
      v[j] = sub + j * G < E ? v[j] : -__builtin_huge_valf();
  }
}

// The top K of each group's token from its loaded keys.  Every lane of the
// wave must call this (it uses wave-wide ballots and reductions).  ent: the
// wave's lds_entries_per_wave<G>() LDS entries.  renorm: weights over the K
// chosen, else over all E.
template <int G, int C, bool FULL>
__device__ __forceinline__ void select(const float (&v)[C], int sub, int E,
                                       int K, int renorm, uint64_t *ent_wave,
                                       Picks &p) {
  constexpr int kCap = 2 * G;        // LDS entries per group
  constexpr int kStride = kCap + 2;  // padded: groups start on other banks
  float lmax = v[0];
#pragma unroll
  for (int j = 1; j < C; ++j) lmax = fmaxf(lmax, v[j]);  // v_max3_f32
  constexpr int kRows = G / 16;
  const int kk = (K + kRows - 1) / kRows;  // <= 16, as K <= G
  const float theta = across_rows_f<G, false>(row_kth_largest(lmax, kk));
  const float mx = across_rows_f<G, true>(row_reduce_f<true>(lmax));

  int cnt = 0;
#pragma unroll
  for (int j = 0; j < C; ++j) cnt += v[j] >= theta ? 1 : 0;
  const int incl = group_inclusive_scan<G>(cnt);
  // the most candidates of any group in the wave (a group's count is the
  // inclusive sum at its last lane)
  int Mw = 0;
#pragma unroll
  for (int g = 0; g < 64 / G; ++g) {
    const int mg = __builtin_amdgcn_readlane(incl, g * G + G - 1);
    Mw = mg > Mw ? mg : Mw;
  }
  // padding keys are -inf: a theta of -inf would take them in
  const bool fast =
      Mw <= kCap && (FULL || !__any(theta == -__builtin_huge_valf()));

  if (fast) {
    uint64_t *ent = ent_wave + ((threadIdx.x & 63) / G) * kStride;
    ent[sub] = 0ull;
    ent[sub + G] = 0ull;
    wave_lds_sync();
    int pos = incl - cnt;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      if (v[j] >= theta) {
        ent[pos] = cand_key(v[j], sub + j * G);
        ++pos;
      }
    }
    wave_lds_sync();
    const int n = (Mw + 3) & ~3;
    if (Mw <= G) {
      rank_entries<G, false>(ent, sub, n, K, p);
    } else {
      rank_entries<G, true>(ent, sub, n, K, p);
    }
  } else {
    uint32_t key[C];
#pragma unroll
    for (int j = 0; j < C; ++j)
      key[j] = sub + j * G < E ? order_bits(v[j]) : 0u;
    const uint32_t th = order_bits(theta);
    uint64_t cmask = 0;  // bit j: key j is a candidate
#pragma unroll
    for (int j = 0; j < C; ++j)
      cmask |= (key[j] != 0u && key[j] >= th) ? (1ull << j) : 0ull;
    Cache cache;
    cache.lk = 0u;
    cache.lp = 0;
    cache.fill<C>(key, cmask, true);
    p.on0 = false;
    p.on1 = false;
    p.r0 = sub;
    p.e0 = 0;
    p.l0 = 0.0f;
    p.r1 = 0;
    p.e1 = 0;
    p.l1 = 0.0f;
    for (int k = 0; k < K; ++k) {
      const uint32_t head = cache.n > 0 ? cache.key[0] : 0u;
      const uint32_t m = group_max<G>(head);
      const uint32_t cand = (cache.n > 0 && head == m)
                                ? (uint32_t)(sub + cache.pos[0] * G)
                                : 0xFFFFFFFFu;
      const uint32_t win = group_min<G>(cand);
      if (sub == k) {
        p.on0 = true;
        p.e0 = (int)win;
        p.l0 = from_order_bits(m);
      }
      if (cand == win) cache.pop();  // the one lane holding the winner
      const bool refill = cache.n == 0 && cache.more;
      if (__any(refill)) {
        if (refill) cache.fill<C>(key, cmask, false);
      }
    }
  }

  // Weights in fp64: exp(l_k - l_max) / sum, rounded once to fp32.
  const double dmx = (double)mx;
  const double x0 = p.on0 ? exp((double)p.l0 - dmx) : 0.0;
  const double x1 = p.on1 ? exp((double)p.l1 - dmx) : 0.0;
  double denom = 0.0;
  if (renorm) {
    denom = x0 + x1;
  } else {
    // every logit of the lane is in v (C*G >= E); padding is -inf (exp 0)
#pragma unroll
    for (int j = 0; j < C; ++j) denom += exp((double)v[j] - dmx);
  }
  denom = group_sum_f64<G>(denom);
  p.w0 = (float)(x0 / denom);
  p.w1 = (float)(x1 / denom);
}

}  // namespace gate
}  // namespace moe
