// Top-K gate kernel for gfx950: one group of G lanes per token; the
// selection itself (threshold, compaction, rank) is in gate_core.h.
//
// "Efficient and portable mixture-of-experts communication", section
// "Introdución": the router yields a distribution over experts, the top-K
// scoring experts are kept, and their outputs are averaged with weights taken
// from that distribution.
#include "gate_core.h"

namespace moe {
namespace {

// C keys per lane; FULL: E == G * C (no padding keys, unclamped loads).
template <int G, int C, bool FULL>
__global__ __launch_bounds__(256) void gate_kernel(
    const float *__restrict__ logits, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int T, int E, int K, int renorm) {
  constexpr int kTokensPerBlock = 256 / G;
  __shared__ __align__(16) uint64_t s_ent[4][gate::lds_entries_per_wave<G>()];

  const int sub = threadIdx.x & (G - 1);
  int t = blockIdx.x * kTokensPerBlock + threadIdx.x / G;
  // groups past the last token compute on token T-1 and store nothing, so
  // every lane of a wave runs the DPP reductions (whole waves leave only
  // when the wave's first token is past the end)
  const bool live = t < T;
  if (blockIdx.x * kTokensPerBlock + (threadIdx.x & ~63) / G >= T) return;
  if (!live) t = T - 1;
  float v[C];
  gate::load_keys<G, C, FULL>(logits + (size_t)t * E, sub, E, v);
  gate::pin_keys<G, C, FULL>(sub, E, v);
  gate::Picks p;
  gate::select<G, C, FULL>(v, sub, E, K, renorm, s_ent[threadIdx.x >> 6], p);
  if (live) {
    if (p.on0) {
      topk_idx[(size_t)t * K + p.r0] = p.e0;
      topk_w[(size_t)t * K + p.r0] = p.w0;
    }
    if (p.on1) {
      topk_idx[(size_t)t * K + p.r1] = p.e1;
      topk_w[(size_t)t * K + p.r1] = p.w1;
    }
  }
}

constexpr int kGateWaveTokens = 1024;  // up to here: one wave per token

template <int G, int C>
hipError_t launch_gc(bool full, const float *logits, int32_t *idx, float *w,
                     int T, int E, int K, int renorm, hipStream_t s) {
  constexpr int tpb = 256 / G;
  const int grid = (T + tpb - 1) / tpb;
  if (full) {
    hipLaunchKernelGGL((gate_kernel<G, C, true>), dim3(grid), dim3(256), 0, s,
                       logits, idx, w, T, E, K, renorm);
  } else {
    hipLaunchKernelGGL((gate_kernel<G, C, false>), dim3(grid), dim3(256), 0,
                       s, logits, idx, w, T, E, K, renorm);
  }
  return hipGetLastError();
}

// Keys per lane: 1, 2, 4, 8, 16, 28 (Kimi K2's E = 896 over 32 lanes), 32;
// with 64 lanes also 48 and 64.
template <int G>
hipError_t launch_g(int C, bool full, const float *logits, int32_t *idx,
                    float *w, int T, int E, int K, int renorm,
                    hipStream_t s) {
  switch (C) {
    case 1: return launch_gc<G, 1>(full, logits, idx, w, T, E, K, renorm, s);
    case 2: return launch_gc<G, 2>(full, logits, idx, w, T, E, K, renorm, s);
    case 4: return launch_gc<G, 4>(full, logits, idx, w, T, E, K, renorm, s);
    case 8: return launch_gc<G, 8>(full, logits, idx, w, T, E, K, renorm, s);
    case 16: return launch_gc<G, 16>(full, logits, idx, w, T, E, K, renorm, s);
    case 28: return launch_gc<G, 28>(full, logits, idx, w, T, E, K, renorm, s);
    case 32: return launch_gc<G, 32>(full, logits, idx, w, T, E, K, renorm, s);
    default: break;
  }
  if constexpr (G == 64) {
    switch (C) {
      case 48: return launch_gc<G, 48>(full, logits, idx, w, T, E, K, renorm, s);
      case 64: return launch_gc<G, 64>(full, logits, idx, w, T, E, K, renorm, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

int keys_per_lane(int need) {
  static const int kC[] = {1, 2, 4, 8, 16, 28, 32, 48, 64};
  for (int c : kC)
    if (c >= need) return c;
  return 0;
}

}  // namespace

hipError_t launch_gate(const moe_cfg &c, const float *logits,
                       int32_t *topk_idx, float *topk_w, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  // The narrowest group with at most 32 keys per lane and K <= G/2: narrow
  // groups share the per-wave work among 64/G tokens, and with G >= 2K the
  // threshold (the ceil(K/rows)-th largest lane maximum of each row) leaves
  // few candidates.  With few tokens (at most one wave per SIMD at G = 64)
  // the kernel is bound by one wave's latency instead, and a whole wave per
  // token, with fewer keys per lane, is faster.
  int G = 16;
  while (G < 64 && ((c.E + G - 1) / G > 32 || 2 * c.K > G)) G <<= 1;
  if (c.T <= kGateWaveTokens) G = 64;
  const int C = keys_per_lane((c.E + G - 1) / G);  // E <= 4096: C <= 64
  const bool full = c.E == G * C;
  const int renorm = (c.flags & MOE_F_NO_RENORM) ? 0 : 1;
  switch (G) {
    case 16: return launch_g<16>(C, full, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    case 32: return launch_g<32>(C, full, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    case 64: return launch_g<64>(C, full, logits, topk_idx, topk_w, c.T, c.E, c.K, renorm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
