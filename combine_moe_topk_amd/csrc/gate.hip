// Top-K gate for gfx950.
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
// the group holds the logits of experts sub, sub+G, sub+2G, ... as 32-bit
// order-preserving keys (larger key = larger logit) and a sorted cache of its
// D best (key, position) pairs, ordered by key descending, position
// ascending.  A round takes the group maximum of the cache heads, then the
// group minimum of the expert indices holding it, so "larger logit, then
// lower index" wins; the winning lane pops its head.  A lane whose cache runs
// empty refills it with the D best pairs strictly after the last one it gave
// out (in the same order), so no key is ever cleared; refills run under a
// wave-uniform branch and are rare (a lane empties only after D wins).
// Group reductions are DPP inside 16-lane rows (quad_perm, half-mirror,
// mirror: every lane of the row ends with the row's result) and readlane
// across rows, with no LDS permutes.  G is the smallest width that keeps at
// most 64 keys per lane and K <= G (the reductions are then shared by the
// 64/G tokens of a wave).
#include "moe_internal.h"

namespace moe {
namespace {

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

template <int G>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
  return v;
}

// The K-th largest of the 16 values of a DPP row (each lane's own value;
// equal values ordered by lane), in every lane of the row: each lane counts
// the lanes whose value ranks before its own, reading them one rotation at
// a time (row_ror), and the lane of rank K-1 gives its value.
template <int R>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x120 + R,
                                               0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t row_kth_largest(uint32_t v, int K) {
  const int me = threadIdx.x & 15;
  int rank = 0;
#define MOE_RANK_STEP(R)                                              \
  {                                                                   \
    const uint32_t o = row_ror<R>(v);                                 \
    const int from = (int)row_ror<R>((uint32_t)me); /* o's lane */    \
    rank += (o > v || (o == v && from < me)) ? 1 : 0;                 \
  }
  MOE_RANK_STEP(1) MOE_RANK_STEP(2) MOE_RANK_STEP(3) MOE_RANK_STEP(4)
  MOE_RANK_STEP(5) MOE_RANK_STEP(6) MOE_RANK_STEP(7) MOE_RANK_STEP(8)
  MOE_RANK_STEP(9) MOE_RANK_STEP(10) MOE_RANK_STEP(11) MOE_RANK_STEP(12)
  MOE_RANK_STEP(13) MOE_RANK_STEP(14) MOE_RANK_STEP(15)
#undef MOE_RANK_STEP
  return group_min<16>(rank == K - 1 ? v : 0xFFFFFFFFu);
}

constexpr int kCache = 4;  // D: cached (key, position) pairs per lane

// Sorted cache of a lane's best keys (key descending, position ascending).
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
  // wave-uniform branch), so the sorted inserts run only for positions
  // that hold one somewhere in the wave.
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

// C keys per lane.  Keys of experts >= E are 0, below every real key (the
// smallest finite logit has key 0x00800000), and never enter a cache.
template <int G, int C>
__global__ __launch_bounds__(256) void gate_kernel(
    const float *__restrict__ logits, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int T, int E, int K, int renorm) {
  constexpr int kTokensPerBlock = 256 / G;
  const int sub = threadIdx.x & (G - 1);
  int t = blockIdx.x * kTokensPerBlock + threadIdx.x / G;
  // groups past the last token compute on token T-1 and store nothing, so
  // every lane of a wave runs the DPP reductions (whole waves leave only
  // when the wave's first token is past the end)
  const bool live = t < T;
  if (blockIdx.x * kTokensPerBlock + (threadIdx.x & ~63) / G >= T) return;
  if (!live) t = T - 1;
  const float *row = logits + (size_t)t * E;

  // Clamped loads, all C issued before the first use.  The empty asm takes
  // every loaded value as an operand, so each load's result is used
  // unconditionally and the compiler cannot move a load into the branch of
  // the padding select below (where it would wait for each load in turn:
  // C memory round trips instead of one).
  float v[C];
#pragma unroll
  for (int j = 0; j < C; ++j) v[j] = row[min(sub + j * G, E - 1)];
#pragma unroll
  for (int j = 0; j < C; ++j) asm volatile("" : "+v"(v[j]));
  uint32_t key[C];
#pragma unroll
  for (int j = 0; j < C; ++j)
    key[j] = sub + j * G < E ? order_bits(v[j]) : 0u;
  // Candidates: keys at or above a threshold theta that at least K keys of
  // the token reach, so the K best are all candidates.  theta is the K-th
  // largest of the G lane maxima (16-lane groups) or their minimum (K = G,
  // or wider groups): at least K lanes hold a key >= theta.  Padding keys
  // (0) are never candidates.
  uint32_t lane_max = 0u;
#pragma unroll
  for (int j = 0; j < C; ++j) lane_max = key[j] > lane_max ? key[j] : lane_max;
  uint32_t theta;
  if constexpr (G == 16) {
    theta = K < 16 ? row_kth_largest(lane_max, K) : group_min<16>(lane_max);
  } else {
    theta = group_min<G>(lane_max);
  }
  uint64_t cmask = 0;  // bit j: key j is a candidate
#pragma unroll
  for (int j = 0; j < C; ++j)
    cmask |= (key[j] != 0u && key[j] >= theta) ? (1ull << j) : 0ull;
  Cache cache;
  cache.lk = 0u;
  cache.lp = 0;
  cache.fill<C>(key, cmask, true);

  int my_e = 0;
  float my_l = 0.0f;
  for (int k = 0; k < K; ++k) {
    const uint32_t head = cache.n > 0 ? cache.key[0] : 0u;
    const uint32_t m = group_max<G>(head);
    const uint32_t cand = (cache.n > 0 && head == m)
                              ? (uint32_t)(sub + cache.pos[0] * G)
                              : 0xFFFFFFFFu;
    const uint32_t win = group_min<G>(cand);
    if (sub == k) {
      my_e = (int)win;
      my_l = from_order_bits(m);
    }
    if (cand == win) cache.pop();  // the one lane holding the winner
    const bool refill = cache.n == 0 && cache.more;
    if (__any(refill)) {
      if (refill) cache.fill<C>(key, cmask, false);
    }
  }

  // Weights in fp64: exp(l_k - l_max) / sum, rounded once to fp32.
  const double mx = (double)__shfl(my_l, 0, G);
  const double ex = (sub < K) ? exp((double)my_l - mx) : 0.0;
  double denom = 0.0;
  if (renorm) {
    denom = ex;
  } else {
    // every logit of the lane is in its keys (C*G >= E); -0.0 came back
    // as +0.0, which gives the same exp(l - max)
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (sub + j * G < E) denom += exp((double)from_order_bits(key[j]) - mx);
  }
  denom = group_sum_f64<G>(denom);

  if (live && sub < K) {
    topk_idx[(size_t)t * K + sub] = my_e;
    topk_w[(size_t)t * K + sub] = (float)(ex / denom);
  }
}

constexpr int kGateWaveTokens = 1024;  // up to here: one wave per token

int pow2_ceil(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

template <int G, int C>
hipError_t launch_gc(const float *logits, int32_t *idx, float *w, int T,
                     int E, int K, int renorm, hipStream_t s) {
  constexpr int tpb = 256 / G;
  const int grid = (T + tpb - 1) / tpb;
  hipLaunchKernelGGL((gate_kernel<G, C>), dim3(grid), dim3(256), 0, s,
                     logits, idx, w, T, E, K, renorm);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(int C, const float *logits, int32_t *idx, float *w,
                    int T, int E, int K, int renorm, hipStream_t s) {
  switch (C) {
    case 1: return launch_gc<G, 1>(logits, idx, w, T, E, K, renorm, s);
    case 2: return launch_gc<G, 2>(logits, idx, w, T, E, K, renorm, s);
    case 4: return launch_gc<G, 4>(logits, idx, w, T, E, K, renorm, s);
    case 8: return launch_gc<G, 8>(logits, idx, w, T, E, K, renorm, s);
    case 16: return launch_gc<G, 16>(logits, idx, w, T, E, K, renorm, s);
    case 32: return launch_gc<G, 32>(logits, idx, w, T, E, K, renorm, s);
    case 48: return launch_gc<G, 48>(logits, idx, w, T, E, K, renorm, s);
    case 56: return launch_gc<G, 56>(logits, idx, w, T, E, K, renorm, s);
    case 64: return launch_gc<G, 64>(logits, idx, w, T, E, K, renorm, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gate(const moe_cfg &c, const float *logits,
                       int32_t *topk_idx, float *topk_w, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  // smallest group with at most 64 keys per lane and K <= G: with 4 or
  // more waves per SIMD the kernel is bound by instruction issue, and narrow
  // groups share the selection's reductions among more tokens.  With few
  // tokens (at most one wave per SIMD at G = 64) it is bound by one wave's
  // latency instead, and a whole wave per token, with 4x fewer keys per
  // lane, is faster: 7.5 against 10.8 us for 128 tokens of the DeepSeek-V3
  // shape, measured on MI355X.
  int G = 16;
  while (G < 64 && ((c.E + G - 1) / G > 64 || G < c.K)) G <<= 1;
  if (c.T <= kGateWaveTokens) G = 64;
  const int need = (c.E + G - 1) / G;  // keys per lane, <= 64
  // keys per lane: a power of two up to 32, then 48, 56 or 64 (56 is the
  // Kimi K2 shape, E = 896 over 16 lanes: no dead key slots)
  int C = need <= 32 ? pow2_ceil(need) : (need <= 48 ? 48 : (need <= 56 ? 56 : 64));
  if (C < 1) C = 1;
  const int renorm = (c.flags & MOE_F_NO_RENORM) ? 0 : 1;
  switch (G) {
    case 16: return launch_g<16>(C, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    case 32: return launch_g<32>(C, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    case 64: return launch_g<64>(C, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
