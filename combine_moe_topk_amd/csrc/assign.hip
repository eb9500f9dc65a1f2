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
// One thread per token: the per-token work is integer and bitmask logic.
// A prep kernel turns the replica map holds[G][E] into one node bitmask per
// expert and one rank bitmask per (expert, node).  The cover search runs over
// the nodes that hold some remote expert of the token only (a minimal cover
// never contains another node), with Gosper's next-combination so masks come
// in (popcount, value) order and the first feasible mask is the answer;
// nodes forced by single-node experts are taken before the search.
#include "moe_internal.h"

namespace moe {
namespace {

// Per expert: the nodes holding it, and per (expert, node) the ranks of
// that node holding it (bit j = rank node*per_node + j; per_node <= 64).
__global__ void expert_tables_kernel(const uint8_t *__restrict__ holds, int E,
                                     int G, int N, int per_node,
                                     uint64_t *__restrict__ nodes,
                                     uint64_t *__restrict__ rank_bits) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  uint64_t m = 0;
  for (int n = 0; n < N; ++n) {
    uint64_t rb = 0;
    for (int j = 0; j < per_node; ++j)
      if (holds[(size_t)(n * per_node + j) * E + e]) rb |= 1ull << j;
    rank_bits[(size_t)e * N + n] = rb;
    if (rb) m |= 1ull << n;
  }
  nodes[e] = m;
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

// KT >= K (slots k >= K are ignored); per_node <= 64.
template <int KT>
__global__ __launch_bounds__(64) void assign_kernel(
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ src_rank,
    const uint64_t *__restrict__ enodes, const uint64_t *__restrict__ rbits,
    const uint32_t *__restrict__ u_node, const uint32_t *__restrict__ u_rank,
    int32_t *__restrict__ assign_rank, uint64_t *__restrict__ remote_mask,
    int T, int E, int K, int G, int N, int32_t *__restrict__ err) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int per_node = G / N;
  const int sr = src_rank[t];
  int bad = 0;
  if ((unsigned)sr >= (unsigned)G) bad |= MOE_DEVERR_SRC_RANK;
  const int sn = bad ? 0 : sr / per_node;
  const uint64_t self = 1ull << sn;

  uint64_t m[KT];
  uint32_t in_u = 0;  // bit k: expert k has no replica on the source node
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    m[k] = 0;
    if (k < K) {
      const int e = topk_idx[(size_t)t * K + k];
      uint64_t nodes = 0;
      if ((unsigned)e >= (unsigned)E) {
        bad |= MOE_DEVERR_EXPERT_RANGE;
      } else {
        nodes = enodes[e];
        if (nodes == 0) bad |= MOE_DEVERR_NO_REPLICA;
      }
      m[k] = nodes & ~self;
      if (!(nodes & self)) in_u |= 1u << k;
    }
  }
  if (bad) {
    atomicOr(err, bad);
    for (int k = 0; k < K; ++k) assign_rank[(size_t)t * K + k] = -1;
    remote_mask[t] = 0;
    return;
  }

  // Step 1: smallest cover of the remote experts, by (popcount, value).
  // A remote expert held by one remote node forces that node into every
  // cover: those nodes (forced) are taken first, and only the experts they
  // leave uncovered are searched, over the nodes holding them.  Forced and
  // searched nodes are disjoint, so (popcount, value) order of the searched
  // part is the order of the whole mask.  Subsets of the searched nodes are
  // enumerated as M-bit numbers with Gosper's hack; expanding keeps the
  // value order.
  uint64_t forced = 0;
#pragma unroll
  for (int k = 0; k < KT; ++k)
    if (((in_u >> k) & 1) && __popcll(m[k]) == 1) forced |= m[k];
  uint32_t left = 0;  // remote experts the forced nodes do not cover
  uint64_t uni = 0;
#pragma unroll
  for (int k = 0; k < KT; ++k)
    if (((in_u >> k) & 1) && !(m[k] & forced)) {
      left |= 1u << k;
      uni |= m[k];
    }
  uint64_t best = forced;
  if (left) {
    const int M = __popcll(uni);  // <= 63: the source node's bit is clear
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
          if (((left >> k) & 1) && !(b & m[k])) ok = false;
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
  remote_mask[t] = best;

  // node, then rank, for every slot (expert and node mask re-read: cache
  // hits, and the loop needs no per-slot arrays)
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    const size_t i = (size_t)t * K + k;
    const int e = topk_idx[i];
    int node = sn;
    if ((in_u >> k) & 1) {
      const uint64_t cand = best & enodes[e] & ~self;
      node = nth_bit(cand, pick(u_node[i], __popcll(cand)));
    }
    const uint64_t rb = rbits[(size_t)e * N + node];
    assign_rank[i] =
        node * per_node + nth_bit(rb, pick(u_rank[i], __popcll(rb)));
  }
}

}  // namespace

size_t assign_ws_bytes(const moe_cfg &c) {
  const size_t tables = (size_t)c.E * 8 + (size_t)c.E * c.N * 8;
  return kWsHeader + ((tables + 255) & ~(size_t)255);
}

bool assign_ok(const moe_cfg &c) { return c.R / c.N <= 64; }

hipError_t launch_assign(const moe_cfg &c, const int32_t *topk_idx,
                         const int32_t *src_rank, const uint8_t *holds,
                         const uint32_t *u_node, const uint32_t *u_rank,
                         int32_t *assign_rank, uint64_t *remote_mask, void *ws,
                         hipStream_t stream) {
  int32_t *err = (int32_t *)ws;
  uint64_t *enodes = (uint64_t *)((char *)ws + kWsHeader);
  uint64_t *rbits = enodes + c.E;
  const int per_node = c.R / c.N;
  hipLaunchKernelGGL(expert_tables_kernel, dim3((c.E + 255) / 256),
                     dim3(256), 0, stream, holds, c.E, c.R, c.N, per_node,
                     enodes, rbits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || c.T == 0) return e;
  // one thread per token, 64-thread workgroups: T/64 waves spread over the
  // CUs (256-thread workgroups would leave most CUs idle at T = 16K)
  const dim3 grid((c.T + 63) / 64), block(64);
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
