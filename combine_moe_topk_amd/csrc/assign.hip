// Communication-aware task assignment for gfx950.
//
// "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
// Training", Section 3.3: a token's selected experts that have a replica on
// its source node run there; the others get the smallest set of remote nodes
// covering them (masks of equal size: the smallest value), a random covering
// node each, then a uniform replica rank inside that node.  Random choices
// come in as uint32 draws u and pick entry floor(u * c / 2^32) of c
// candidates in ascending order.
//
// One wave per token.  Lane k < K holds slot k: its expert, the nodes
// holding that expert and, at the end, its node and rank draws, so the
// per-slot work and its loads run side by side.  A prep kernel turns the
// replica map holds[G][E] into one node bitmask per expert and one rank
// bitmask per (expert, node).  Nodes forced by single-node experts are taken
// first; the remaining experts' candidate nodes (M of them; a minimal cover
// never contains another node) are covered by the smallest subset, smallest
// value first.  Up to M = 12 the wave tests all 2^M subsets, 64 at a time
// (lane j takes subset base + j), and a wave minimum of (popcount, index)
// over the feasible ones picks the same subset as enumerating them in that
// order; above it the wave walks them in order with Gosper's
// next-combination.  The subset index maps to nodes in ascending order, so
// index order is node-mask order.  (A thread per token, as before, left one
// wave per CU at 16K tokens and each wave waited for its slowest token's
// search: 32 us against 8 us for the DeepSeek-V3 shape.)
#include "moe_internal.h"

namespace moe {
namespace {

// Per expert: the nodes holding it, and per (expert, node) the ranks of
// that node holding it (bit j = rank node*per_node + j; per_node <= 64).
// One wave per expert, lane n < N for node n (N <= 64): the lane gathers
// its node's per_node flags, and a ballot of the non-empty lanes is the
// expert's node mask.
__global__ __launch_bounds__(256) void expert_tables_kernel(
    const uint8_t *__restrict__ holds, int E, int N, int per_node,
    uint64_t *__restrict__ nodes, uint64_t *__restrict__ rank_bits) {
  const int lane = threadIdx.x % kWave;
  const int e = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (e >= E) return;  // one expert per wave: uniform exit
  uint64_t rb = 0;
  if (lane < N) {
    const uint8_t *h = holds + (size_t)lane * per_node * E + e;
    int j = 0;
    for (; j + 8 <= per_node; j += 8) {  // 8 independent loads at a time
      uint8_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = h[(size_t)(j + q) * E];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (v[q]) rb |= 1ull << (j + q);
    }
    for (; j < per_node; ++j)
      if (h[(size_t)j * E]) rb |= 1ull << j;
    rank_bits[(size_t)e * N + lane] = rb;
  }
  const uint64_t m = __ballot(rb != 0);
  if (lane == 0) nodes[e] = m;
}

__device__ __forceinline__ int pick(uint32_t u, int c) {
  return (int)(((uint64_t)u * (uint64_t)c) >> 32);
}

// j-th set bit (ascending) of m; m has more than j bits
__device__ __forceinline__ int nth_bit(uint64_t m, int j) {
#pragma unroll 1
  for (; j > 0; --j) m &= m - 1;
  return __builtin_ctzll(m);
}

// the subset of `uni` whose members are selected by the low bits of c
// (bit j of c picks the j-th lowest member of uni)
__device__ __forceinline__ uint64_t expand(uint64_t c, uint64_t uni) {
  uint64_t b = 0;
#pragma unroll 1
  for (; c; c >>= 1) {
    const uint64_t low = uni & (~uni + 1);
    if (c & 1) b |= low;
    uni ^= low;
  }
  return b;
}

// 64-bit value of lane `src`, wave-uniform.
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int src) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1)
    v = min(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v |= __shfl_xor(v, off);
  return v;
}

constexpr int kParallelCoverM = 12;  // test all 2^M subsets up to this M

// One wave per token; KT >= K (<= 32) slots, lane k < K holds slot k.
template <int KT>
__global__ __launch_bounds__(256) void assign_kernel(
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ src_rank,
    const uint64_t *__restrict__ enodes, const uint64_t *__restrict__ rbits,
    const uint32_t *__restrict__ u_node, const uint32_t *__restrict__ u_rank,
    int32_t *__restrict__ assign_rank, uint64_t *__restrict__ remote_mask,
    int T, int E, int K, int G, int N, int32_t *__restrict__ err) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // one token per wave: uniform exit
  const int per_node = G / N;
  const int sr = src_rank[t];
  int bad = (unsigned)sr >= (unsigned)G ? MOE_DEVERR_SRC_RANK : 0;
  const int sn = bad ? 0 : sr / per_node;
  const uint64_t self = 1ull << sn;
  const bool mine = lane < K;  // this lane holds a slot
  const size_t i = (size_t)t * K + (mine ? lane : 0);
  int e = 0;
  uint64_t nodes = 0;
  uint32_t un = 0, ur = 0;
  if (mine) {  // all of the slot's loads go out together
    e = topk_idx[i];
    un = u_node[i];
    ur = u_rank[i];
    if ((unsigned)e >= (unsigned)E) {
      bad |= MOE_DEVERR_EXPERT_RANGE;
    } else {
      nodes = enodes[e];
      if (nodes == 0) bad |= MOE_DEVERR_NO_REPLICA;
    }
  }
  bad = wave_or(bad);
  if (bad) {
    if (lane == 0) {
      atomicOr(err, bad);
      remote_mask[t] = 0;
    }
    if (mine) assign_rank[i] = -1;
    return;
  }
  const uint64_t m = nodes & ~self;  // remote nodes holding the expert
  const bool remote = mine && !(nodes & self);
  const uint32_t in_u = (uint32_t)__ballot(remote);  // K <= 32
  uint64_t mk[KT];  // every slot's remote nodes, wave-uniform
#pragma unroll
  for (int k = 0; k < KT; ++k) mk[k] = readlane64(m, k);

  // Nodes forced by experts held on one remote node only, then the experts
  // they leave uncovered and those experts' candidate nodes.
  uint64_t forced = 0;
#pragma unroll
  for (int k = 0; k < KT; ++k)
    if (((in_u >> k) & 1) && __popcll(mk[k]) == 1) forced |= mk[k];
  uint32_t left = 0;
  uint64_t uni = 0;
#pragma unroll
  for (int k = 0; k < KT; ++k)
    if (((in_u >> k) & 1) && !(mk[k] & forced)) {
      left |= 1u << k;
      uni |= mk[k];
    }
  uint64_t best = forced;
  if (left) {
    const int M = __popcll(uni);  // <= 63: the source node's bit is clear
    if (M <= kParallelCoverM) {
      uint32_t key = 0xFFFFFFFFu;  // (popcount << 16) | index, feasible only
      for (int base = 0; base < (1 << M); base += kWave) {
        const uint32_t c = (uint32_t)(base + lane);
        const uint64_t b = expand(c, uni);
        bool ok = c < (1u << M);
#pragma unroll
        for (int k = 0; k < KT; ++k)
          if (((left >> k) & 1) && !(b & mk[k])) ok = false;
        if (ok) key = min(key, ((uint32_t)__popc(c) << 16) | c);
      }
      best = forced | expand(wave_min(key) & 0xFFFFu, uni);
    } else {
      // subsets in (popcount, value) order, Gosper's next-combination; the
      // values are wave-uniform, so every lane walks the same sequence
      bool found = false;
#pragma unroll 1
      for (int p = 1; p <= M && !found; ++p) {
        const uint64_t end = 1ull << M;
#pragma unroll 1
        for (uint64_t c = (1ull << p) - 1; c < end;) {
          const uint64_t b = expand(c, uni);
          bool ok = true;
#pragma unroll
          for (int k = 0; k < KT; ++k)
            if (((left >> k) & 1) && !(b & mk[k])) ok = false;
          if (ok) {
            best = forced | b;
            found = true;
            break;
          }
          const uint64_t low = c & (~c + 1);
          const uint64_t ripple = c + low;
          c = ripple | (((ripple ^ c) >> 2) >> __builtin_ctzll(low));
        }
      }
    }
  }
  if (lane == 0) remote_mask[t] = best;

  // this lane's slot: a covering node for a remote expert (the source node
  // otherwise), then a replica rank inside that node
  if (!mine) return;
  int node = sn;
  if (remote) {
    const uint64_t cand = best & m;
    node = nth_bit(cand, pick(un, __popcll(cand)));
  }
  const uint64_t rb = rbits[(size_t)e * N + node];
  assign_rank[i] = node * per_node + nth_bit(rb, pick(ur, __popcll(rb)));
}

}  // namespace

size_t assign_ws_bytes(const moe_cfg &c) {
  const size_t tables = (size_t)c.E * 8 + (size_t)c.E * c.N * 8;
  return kWsHeader + ((tables + 255) & ~(size_t)255);
}

// At most kMaxAssignNodes nodes: the minimum cover walks subsets of the up
// to N - 1 remote candidate nodes in size order, so one token may test up to
// 2^(N-1) of them ("Cobalt: Leveraging Expert Co-activation for Efficient
// Distributed MoE Training", Section 3.3, gives the search this cost and
// takes the expert-parallel degree to be small).  With N <= 24 a wave tests
// at most 2^23 subsets and always finishes; a larger N is refused on the
// host before anything is enqueued.
bool assign_ok(const moe_cfg &c) {
  return c.N <= kMaxAssignNodes && c.R / c.N <= 64;
}

hipError_t launch_assign(const moe_cfg &c, const int32_t *topk_idx,
                         const int32_t *src_rank, const uint8_t *holds,
                         const uint32_t *u_node, const uint32_t *u_rank,
                         int32_t *assign_rank, uint64_t *remote_mask, void *ws,
                         hipStream_t stream) {
  int32_t *err = (int32_t *)ws;
  uint64_t *enodes = (uint64_t *)((char *)ws + kWsHeader);
  uint64_t *rbits = enodes + c.E;
  const int per_node = c.R / c.N;
  hipLaunchKernelGGL(expert_tables_kernel, dim3((c.E + 3) / 4), dim3(256), 0,
                     stream, holds, c.E, c.N, per_node, enodes, rbits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.T == 0) return e;
  const dim3 grid((c.T + 3) / 4), block(256);  // one wave per token
#define MOE_ASSIGN(KT_)                                                     \
  hipLaunchKernelGGL((assign_kernel<KT_>), grid, block, 0, stream, topk_idx, \
                     src_rank, enodes, rbits, u_node, u_rank, assign_rank,  \
                     remote_mask, c.T, c.E, c.K, c.R, c.N, err)
  if (c.K <= 2) MOE_ASSIGN(2);
  else if (c.K <= 4) MOE_ASSIGN(4);
  else if (c.K <= 8) MOE_ASSIGN(8);
  else if (c.K <= 16) MOE_ASSIGN(16);
  else MOE_ASSIGN(32);
#undef MOE_ASSIGN
  return hipGetLastError();
}

}  // namespace moe
