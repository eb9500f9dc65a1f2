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
// Layout: a group of G lanes (G a power of two, 8..64) owns one token.  Lane
// `sub` of the group holds the logits of experts sub, sub+G, sub+2G, ... as
// 64-bit keys (order-preserving logit bits << 32 | ~expert), so one unsigned
// max picks "larger logit, then lower index".  K rounds of (per-lane max,
// butterfly max over the group, winner cleared) select the experts in
// descending order; lane k of the group keeps round k's winner.  Row loads are
// coalesced: G consecutive floats per group per load.
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

template <int G, int C>
__global__ __launch_bounds__(256) void gate_kernel(
    const float *__restrict__ logits, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int T, int E, int K, int renorm) {
  constexpr int kTokensPerBlock = 256 / G;
  const int sub = threadIdx.x & (G - 1);
  const int t = blockIdx.x * kTokensPerBlock + threadIdx.x / G;
  if (t >= T) return;  // whole groups leave together
  const float *row = logits + (size_t)t * E;

  uint64_t key[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int e = sub + j * G;
    key[j] = 0;  // below every real key
    if (e < E)
      key[j] = ((uint64_t)order_bits(row[e]) << 32) |
               (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
  }

  int my_e = 0;
  float my_l = 0.0f;
  for (int k = 0; k < K; ++k) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < C; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
      const uint64_t o = __shfl_xor(best, off, G);
      best = o > best ? o : best;
    }
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (key[j] == best) key[j] = 0;  // keys are unique: one owner
    if (sub == k) {
      my_e = (int)(0xFFFFFFFFu - (uint32_t)best);
      my_l = from_order_bits((uint32_t)(best >> 32));
    }
  }

  // Weights in fp64: exp(l_k - l_max) / sum, rounded once to fp32.
  const double m = (double)__shfl(my_l, 0, G);
  const double ex = (sub < K) ? exp((double)my_l - m) : 0.0;
  double denom = 0.0;
  if (renorm) {
    denom = ex;
  } else {
    for (int e = sub; e < E; e += G) denom += exp((double)row[e] - m);
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) denom += __shfl_xor(denom, off, G);

  if (sub < K) {
    topk_idx[(size_t)t * K + sub] = my_e;
    topk_w[(size_t)t * K + sub] = (float)(ex / denom);
  }
}

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
    default: break;
  }
  if constexpr (G == 64) {
    switch (C) {
      case 16: return launch_gc<64, 16>(logits, idx, w, T, E, K, renorm, s);
      case 32: return launch_gc<64, 32>(logits, idx, w, T, E, K, renorm, s);
      case 64: return launch_gc<64, 64>(logits, idx, w, T, E, K, renorm, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gate(const moe_cfg &c, const float *logits,
                       int32_t *topk_idx, float *topk_w, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  // About 8 logits per lane; a group is never narrower than K.
  int G = pow2_ceil((c.E + 7) / 8);
  G = G < 8 ? 8 : (G > 64 ? 64 : G);
  const int gk = pow2_ceil(c.K);
  if (G < gk) G = gk;
  const int C = pow2_ceil((c.E + G - 1) / G);
  const int renorm = (c.flags & MOE_F_NO_RENORM) ? 0 : 1;
  switch (G) {
    case 8: return launch_g<8>(C, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    case 16: return launch_g<16>(C, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    case 32: return launch_g<32>(C, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    case 64: return launch_g<64>(C, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
