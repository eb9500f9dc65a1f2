// Top-K gate kernels for gfx950: one group of G lanes per token; the
// selection itself (threshold, compaction, rank) is in gate_core.h.  The
// gate kernel writes the picks; the gate-count kernel, for the fused call,
// also writes the dispatch layout's per-tile counts in the same launch.
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
  if ((int)blockIdx.x * kTokensPerBlock + (int)(threadIdx.x & ~63u) / G >= T)
    return;
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

// The gate and the layout's count pass in one launch, for the fused call:
// workgroup b owns layout tile b (64 * passes tokens, 16 lanes a token, 64
// tokens a pass), runs the gate of each of its tokens as gate_kernel<16, C,
// FULL> does and stores the picks, then, instead of a separate count launch
// reading the ids back, sets the bits of its tokens' picks in LDS bitmaps
// (one 64-bit word per pass and expert / rank / node column; setting a bit
// twice is setting it once, so a token counts once in each rank and node
// column) and writes the tile's row of the count table and the tokens'
// node masks.  Same outputs as the gate then the layout count kernel.
template <int C, bool FULL>
__global__ __launch_bounds__(1024) void gate_count_kernel(
    const float *__restrict__ logits, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int T, int E, int K, int renorm, int R, int N,
    uint32_t m_rank, uint32_t m_node, int passes,
    uint64_t *__restrict__ node_mask, int32_t *__restrict__ table) {
  constexpr int G = 16;
  __shared__ __align__(16) uint64_t s_ent[16][gate::lds_entries_per_wave<G>()];
  extern __shared__ uint64_t bm[];  // [passes][cols], then [passes * 64]
  const int cols = E + R + N;
  uint64_t *nm = bm + (size_t)passes * cols;  // node mask of each token
  for (int i = threadIdx.x; i < passes * (cols + 64); i += blockDim.x)
    bm[i] = 0;
  __syncthreads();

  const int sub = threadIdx.x & (G - 1);
  const int j = threadIdx.x / G;  // the thread's token within a pass
  const int t0 = blockIdx.x * passes * 64;
  for (int i = 0; i < passes; ++i) {
    const int base = t0 + i * 64;
    // waves whose tokens are all past the end skip the pass (wave-uniform:
    // the selection synchronises only within the wave)
    if (base + (int)(threadIdx.x & ~63u) / G >= T) continue;
    int t = base + j;
    const bool live = t < T;
    if (!live) t = T - 1;
    float v[C];
    gate::load_keys<G, C, FULL>(logits + (size_t)t * E, sub, E, v);
    gate::pin_keys<G, C, FULL>(sub, E, v);
    gate::Picks p;
    gate::select<G, C, FULL>(v, sub, E, K, renorm, s_ent[threadIdx.x >> 6],
                             p);
    if (!live) continue;
    unsigned long long *row = (unsigned long long *)(bm + (size_t)i * cols);
    const unsigned long long bit = 1ull << j;
    uint64_t nodes = 0;
    for (int d = 0; d < 2; ++d) {
      if (!(d ? p.on1 : p.on0)) continue;
      const int r = d ? p.r1 : p.r0, e = d ? p.e1 : p.e0;
      topk_idx[(size_t)t * K + r] = e;
      topk_w[(size_t)t * K + r] = d ? p.w1 : p.w0;
      const int n = div_small(e, m_node);
      atomicOr(&row[e], bit);
      atomicOr(&row[E + div_small(e, m_rank)], bit);
      atomicOr(&row[E + R + n], bit);
      nodes |= 1ull << n;
    }
    if (nodes) atomicOr((unsigned long long *)&nm[i * 64 + j], nodes);
  }
  __syncthreads();

  int32_t *out = table + (size_t)blockIdx.x * cols;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) {
    int s = 0;
    for (int i = 0; i < passes; ++i) s += __popcll(bm[(size_t)i * cols + c]);
    out[c] = s;
  }
  if (node_mask)
    for (int q = threadIdx.x; q < passes * 64; q += blockDim.x)
      if (t0 + q < T) node_mask[t0 + q] = nm[q];
}

constexpr int kGateWaveTokens = 1024;  // up to here: one wave per token
constexpr int kGateCountMaxPasses = 1;

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

// The narrowest group with at most 32 keys per lane and K <= G/2: narrow
// groups share the per-wave work among 64/G tokens, and with G >= 2K the
// threshold (the ceil(K/rows)-th largest lane maximum of each row) leaves
// few candidates.  With few tokens (at most one wave per SIMD at G = 64)
// the kernel is bound by one wave's latency instead, and a whole wave per
// token, with fewer keys per lane, is faster.
int gate_group(const moe_cfg &c) {
  int G = 16;
  while (G < 64 && ((c.E + G - 1) / G > 32 || 2 * c.K > G)) G <<= 1;
  if (c.T <= kGateWaveTokens) G = 64;
  return G;
}

size_t gate_count_lds(const moe_cfg &c, int passes) {
  return (size_t)passes * (c.E + c.R + c.N + 64) * 8;
}

template <int C>
hipError_t launch_gate_count_c(const moe_cfg &c, bool full, int passes,
                               int nblocks, const float *logits,
                               int32_t *idx, float *w, uint64_t *node_mask,
                               int32_t *table, hipStream_t s) {
  const int renorm = (c.flags & MOE_F_NO_RENORM) ? 0 : 1;
  const uint32_t m_rank = div_magic(c.E / c.R);
  const uint32_t m_node = div_magic(c.E / c.N);
  const size_t lds = gate_count_lds(c, passes);
  if (full) {
    hipLaunchKernelGGL((gate_count_kernel<C, true>), dim3(nblocks),
                       dim3(1024), lds, s, logits, idx, w, c.T, c.E, c.K,
                       renorm, c.R, c.N, m_rank, m_node, passes, node_mask,
                       table);
  } else {
    hipLaunchKernelGGL((gate_count_kernel<C, false>), dim3(nblocks),
                       dim3(1024), lds, s, logits, idx, w, c.T, c.E, c.K,
                       renorm, c.R, c.N, m_rank, m_node, passes, node_mask,
                       table);
  }
  return hipGetLastError();
}

}  // namespace

bool gate_count_ok(const moe_cfg &c) {
  if (c.T <= 0 || gate_group(c) != 16) return false;
  const LayoutGeom g = layout_geom(c);
  const int passes = g.tile_tokens / kWave;
  return g.nblocks > 1 && passes <= kGateCountMaxPasses &&
         gate_count_lds(c, passes) <= (size_t)kLdsBudget;
}

hipError_t launch_gate_count(const moe_cfg &c, const float *logits,
                             int32_t *topk_idx, float *topk_w,
                             uint64_t *node_mask, void *ws,
                             hipStream_t stream) {
  if (!gate_count_ok(c)) return hipErrorInvalidValue;
  const LayoutGeom g = layout_geom(c);
  const int passes = g.tile_tokens / kWave;
  const int C = keys_per_lane((c.E + 15) / 16);
  const bool full = c.E == 16 * C;
  int32_t *table = (int32_t *)((char *)ws + kWsHeader);
  switch (C) {
#define MOE_GC(CC)                                                          \
  case CC:                                                                  \
    return launch_gate_count_c<CC>(c, full, passes, g.nblocks, logits,      \
                                   topk_idx, topk_w, node_mask, table,      \
                                   stream);
    MOE_GC(1) MOE_GC(2) MOE_GC(4) MOE_GC(8) MOE_GC(16) MOE_GC(28) MOE_GC(32)
#undef MOE_GC
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gate(const moe_cfg &c, const float *logits,
                       int32_t *topk_idx, float *topk_w, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int G = gate_group(c);
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
