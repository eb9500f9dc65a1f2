// Node-level two-leg dispatch and hierarchical combine for gfx950.
//
// "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
// Training", Section 1: when several of a token's experts live on one node,
// the token crosses to that node once and is forwarded inside it.  "MoX:
// Efficient MoE Routing on Direct-Connect Topologies", Section 2.5: the
// combine runs the dispatch tree backwards, and a node reduces the expert
// outputs it holds for a token before forwarding one vector to the source.
//
// On one GPU both legs are copies between HBM buffers:
//   leg 1  node_send[node_slot[t,n]] = x[t]          (launch_pack_rows, W=N)
//   leg 2  send[slot_pos[t,k]] = node_send[node_slot[t, node(e(t,k))]]
//   back   part[node_slot[t,n]] = sum_{k on n} w s y[slot_pos[t,k]]  (fp32)
//          out[t] = sum_n part[node_slot[t,n]]                         (fp32)
// node(e) = (e / (E/R)) / (R/N).  Every kernel reads its per-token routing
// into lanes (k < K, n < N) and broadcasts it with readlane, so row
// addresses are scalar; rows move as 16-byte vectors.
#include "moe_internal.h"
#include "row_io.h"

namespace moe {
namespace {

// Wave-uniform set of the nodes a token's valid experts live on.
__device__ __forceinline__ uint64_t node_set(int my_node, int K) {
  uint64_t m = 0;
  for (int k = 0; k < K; ++k) {
    const int n = __builtin_amdgcn_readlane(my_node, k);
    if (n >= 0) m |= 1ull << n;
  }
  return m;
}

// ---- leg 2: one wave per token ----------------------------------------
// For every node n the token reached, the wave loads node_send's row once
// (VPL vectors per lane per pass) and stores it to the send row of every
// slot k whose expert lives on n.
template <int VPL>
__global__ __launch_bounds__(256) void forward_kernel(
    const u32x4 *__restrict__ node_send, const int32_t *__restrict__ node_slot,
    const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ slot_pos,
    u32x4 *__restrict__ send, int T, int K, int N, int E, int per_rank,
    int per_node, int V, int node_rows, int rows) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // one token per wave: uniform exit
  int my_dst = -1, my_node = -1, my_src = -1;
  if (lane < K) {
    const int e = topk_idx[(size_t)t * K + lane];
    const int d = slot_pos[(size_t)t * K + lane];
    if ((unsigned)e < (unsigned)E && (unsigned)d < (unsigned)rows) {
      my_node = (e / per_rank) / per_node;
      my_dst = d;
    }
  }
  if (lane < N) my_src = node_slot[(size_t)t * N + lane];
  const uint64_t nodes = node_set(my_node, K);

  for (int base = 0; base < V; base += kWave * VPL) {
    for (uint64_t m = nodes; m; m &= m - 1) {
      const int n = __builtin_ctzll(m);
      const int src = __builtin_amdgcn_readlane(my_src, n);
      if ((unsigned)src >= (unsigned)node_rows) continue;
      const u32x4 *row = node_send + (size_t)src * V;
      u32x4 v[VPL];
#pragma unroll
      for (int j = 0; j < VPL; ++j) v[j] = row[min(base + j * kWave + lane, V - 1)];
      for (int k = 0; k < K; ++k) {
        if (__builtin_amdgcn_readlane(my_node, k) != n) continue;
        u32x4 *dst = send + (size_t)__builtin_amdgcn_readlane(my_dst, k) * V;
#pragma unroll
        for (int j = 0; j < VPL; ++j) {
          const int i = base + j * kWave + lane;
          if (i < V) dst[i] = v[j];
        }
      }
    }
  }
}

// ---- reverse of leg 2: per-node partial sums --------------------------
// TPT threads own a token (as in the flat combine).  The token's K slots are
// first ordered by (node, k): lane k computes its position in that order,
// and position i is read back with a ballot, so slot, coefficient and node
// of position i are wave-uniform.  Rows are loaded in that order (all K*UPT
// loads of a pass issued before the first FMA) and reduced in one
// segmented pass: when the node changes after position i, the fp32 sum of
// the segment is stored to the node's partial row (rounded once when the
// partial type is bf16).  One pass over the slots keeps the register
// footprint of the flat combine; a loop over nodes would let the compiler
// keep every widened element live across it.
// KT: K rounded up to a power of two (<= 32); slots k >= K are invalid.
template <bool YB, bool PB, int KT, int UPT, int TPT>
__global__ __launch_bounds__(256) void partial_kernel(
    const char *__restrict__ y, const int32_t *__restrict__ slot_pos,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ scale, const int32_t *__restrict__ node_slot,
    char *__restrict__ part, int T, int K, int N, int E, int per_rank,
    int per_node, int U, int rows, int node_rows) {
  const int lane = threadIdx.x % kWave;
  const int tt = threadIdx.x % TPT;
  const int t = blockIdx.x * (256 / TPT) + threadIdx.x / TPT;
  if (t >= T) return;  // whole waves leave together
  const size_t ybytes = (size_t)U * (YB ? 16 : 32);
  const size_t pbytes = (size_t)U * (PB ? 16 : 32);

  int my_slot = 0, my_node = -1, my_src = -1;
  float my_c = 0.0f;
  if (lane < K) {
    const size_t i = (size_t)t * K + lane;
    const int e = topk_idx[i];
    const int s = slot_pos[i];
    if ((unsigned)e < (unsigned)E && (unsigned)s < (unsigned)rows) {
      my_slot = s;
      my_node = (e / per_rank) / per_node;
      my_c = topk_w[i];
      if (scale) my_c *= scale[e];
    }
  }
  if (lane < N) my_src = node_slot[(size_t)t * N + lane];
  // position of slot `lane` in (node, k) order; invalid slots (node -1)
  // come first and are never stored
  int my_pos = 0;
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    const int nk = __builtin_amdgcn_readlane(my_node, k);
    my_pos += (nk < my_node || (nk == my_node && k < lane)) ? 1 : 0;
  }
  int o_slot[KT], o_node[KT];
  float o_c[KT];
#pragma unroll
  for (int i = 0; i < KT; ++i) {
    const uint64_t hit = __ballot(lane < KT && my_pos == i);
    const int k = __builtin_ctzll(hit);
    o_slot[i] = __builtin_amdgcn_readlane(my_slot, k);
    o_node[i] = __builtin_amdgcn_readlane(my_node, k);
    o_c[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_c), k));
  }
  // invalid positions (first in the order, weight 0) re-read the last
  // position's row, which is loaded anyway: loads stay branch-free
#pragma unroll
  for (int i = 0; i < KT - 1; ++i)
    if (o_node[i] < 0) o_slot[i] = o_slot[KT - 1];

  for (int base = 0; base < U; base += TPT * UPT) {
    Unit<YB> u[KT][UPT];
#pragma unroll
    for (int i = 0; i < KT; ++i) {
      const char *row = y + (size_t)o_slot[i] * ybytes;
#pragma unroll
      for (int j = 0; j < UPT; ++j)
        u[i][j].load(row, min(base + j * TPT + tt, U - 1));
    }
    float acc[UPT][8];
#pragma unroll
    for (int j = 0; j < UPT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < KT; ++i) {
#pragma unroll
      for (int j = 0; j < UPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[j][e] = fmaf(o_c[i], u[i][j].get(e), acc[j][e]);
      if (i + 1 < KT && o_node[i + 1] == o_node[i]) continue;
      // end of node o_node[i]'s segment
      const int p = o_node[i] >= 0 ? __builtin_amdgcn_readlane(my_src, o_node[i])
                                   : -1;
      if ((unsigned)p < (unsigned)node_rows) {
        char *prow = part + (size_t)p * pbytes;
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
          const int q = base + j * TPT + tt;
          if (q < U) store_unit<PB>(prow, q, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < UPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
    }
  }
}

// ---- reverse of leg 1: sum of a token's node partials -----------------
// The token's partial rows are taken in batches of NB; a batch's NB*UPT
// loads are issued together (batch entries past the token's last node
// re-read its last row and are not added), then summed in fp32.
constexpr int kNodeBatch = 8;

template <bool PB, bool OB, int UPT, int TPT>
__global__ __launch_bounds__(256) void sum_nodes_kernel(
    const char *__restrict__ part, const int32_t *__restrict__ node_slot,
    char *__restrict__ out, int T, int N, int U, int node_rows) {
  const int lane = threadIdx.x % kWave;
  const int tt = threadIdx.x % TPT;
  const int t = blockIdx.x * (256 / TPT) + threadIdx.x / TPT;
  if (t >= T) return;
  const size_t pbytes = (size_t)U * (PB ? 16 : 32);
  const size_t obytes = (size_t)U * (OB ? 16 : 32);
  int my_src = -1;
  if (lane < N) my_src = node_slot[(size_t)t * N + lane];
  // every wave of the token's group holds the same node_slot entries
  const uint64_t present = __ballot((unsigned)my_src < (unsigned)node_rows);
  char *orow = out + (size_t)t * obytes;

  for (int base = 0; base < U; base += TPT * UPT) {
    float acc[UPT][8];
#pragma unroll
    for (int j = 0; j < UPT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;
    for (uint64_t m = present; m;) {
      // m != 0 here: entry 0 is a present node; later entries repeat the
      // previous one once the set runs out
      int src[kNodeBatch];
      src[0] = __builtin_amdgcn_readlane(my_src, __builtin_ctzll(m));
      m &= m - 1;
      int cnt = 1;
#pragma unroll
      for (int b = 1; b < kNodeBatch; ++b) {
        if (m) {
          src[b] = __builtin_amdgcn_readlane(my_src, __builtin_ctzll(m));
          m &= m - 1;
          cnt = b + 1;
        } else {
          src[b] = src[b - 1];
        }
      }
      Unit<PB> u[kNodeBatch][UPT];
#pragma unroll
      for (int b = 0; b < kNodeBatch; ++b) {
        const char *row = part + (size_t)src[b] * pbytes;
#pragma unroll
        for (int j = 0; j < UPT; ++j)
          u[b][j].load(row, min(base + j * TPT + tt, U - 1));
      }
#pragma unroll
      for (int b = 0; b < kNodeBatch; ++b) {
        if (b >= cnt) break;
#pragma unroll
        for (int j = 0; j < UPT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j][e] += u[b][j].get(e);
      }
    }
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int i = base + j * TPT + tt;
      if (i < U) store_unit<OB>(orow, i, acc[j]);
    }
  }
}

// ---- launch helpers ----------------------------------------------------
template <int VPL>
hipError_t launch_fwd(const moe_cfg &c, const void *node_send,
                      const int32_t *node_slot, const int32_t *topk_idx,
                      const int32_t *slot_pos, void *send, int V,
                      int node_rows, hipStream_t s) {
  const int grid = (c.T + 3) / 4;
  hipLaunchKernelGGL((forward_kernel<VPL>), dim3(grid), dim3(256), 0, s,
                     (const u32x4 *)node_send, node_slot, topk_idx, slot_pos,
                     (u32x4 *)send, c.T, c.K, c.N, c.E, c.E / c.R,
                     c.R / c.N, V, node_rows, c.T * c.K);
  return hipGetLastError();
}

// About 32 16-byte row loads in flight per thread (as in the flat combine).
template <bool YB, int KT>
constexpr int partial_upt() {
  constexpr int per_unit = YB ? 1 : 2;
  constexpr int raw = 32 / (KT * per_unit);
  return raw < 1 ? 1 : (raw > 8 ? 8 : raw);
}

template <bool YB, bool PB, int KT>
hipError_t launch_partial_k(const moe_cfg &c, const void *y,
                            const int32_t *slot_pos, const float *w,
                            const int32_t *idx, const float *scale,
                            const int32_t *node_slot, void *part,
                            int node_rows, hipStream_t s) {
  constexpr int UPT = partial_upt<YB, KT>();
  const int U = c.H / 8;
  if (U <= 64 * UPT) {
    hipLaunchKernelGGL((partial_kernel<YB, PB, KT, UPT, 64>),
                       dim3((c.T + 3) / 4), dim3(256), 0, s, (const char *)y,
                       slot_pos, w, idx, scale, node_slot, (char *)part, c.T,
                       c.K, c.N, c.E, c.E / c.R, c.R / c.N, U, c.T * c.K,
                       node_rows);
  } else {
    hipLaunchKernelGGL((partial_kernel<YB, PB, KT, UPT, 256>), dim3(c.T),
                       dim3(256), 0, s, (const char *)y, slot_pos, w, idx,
                       scale, node_slot, (char *)part, c.T, c.K, c.N, c.E,
                       c.E / c.R, c.R / c.N, U, c.T * c.K, node_rows);
  }
  return hipGetLastError();
}

template <bool YB, bool PB>
hipError_t launch_partial_d(const moe_cfg &c, const void *y,
                            const int32_t *slot_pos, const float *w,
                            const int32_t *idx, const float *scale,
                            const int32_t *node_slot, void *part,
                            int node_rows, hipStream_t s) {
  if (c.K <= 1) return launch_partial_k<YB, PB, 1>(c, y, slot_pos, w, idx, scale, node_slot, part, node_rows, s);
  if (c.K <= 2) return launch_partial_k<YB, PB, 2>(c, y, slot_pos, w, idx, scale, node_slot, part, node_rows, s);
  if (c.K <= 4) return launch_partial_k<YB, PB, 4>(c, y, slot_pos, w, idx, scale, node_slot, part, node_rows, s);
  if (c.K <= 8) return launch_partial_k<YB, PB, 8>(c, y, slot_pos, w, idx, scale, node_slot, part, node_rows, s);
  if (c.K <= 16) return launch_partial_k<YB, PB, 16>(c, y, slot_pos, w, idx, scale, node_slot, part, node_rows, s);
  return launch_partial_k<YB, PB, 32>(c, y, slot_pos, w, idx, scale, node_slot, part, node_rows, s);
}

template <bool PB, bool OB>
hipError_t launch_sum_d(const moe_cfg &c, const void *part,
                        const int32_t *node_slot, void *out, int node_rows,
                        hipStream_t s) {
  constexpr int UPT = 32 / (kNodeBatch * (PB ? 1 : 2));
  const int U = c.H / 8;
  if (U <= 64 * UPT) {
    hipLaunchKernelGGL((sum_nodes_kernel<PB, OB, UPT, 64>),
                       dim3((c.T + 3) / 4), dim3(256), 0, s,
                       (const char *)part, node_slot, (char *)out, c.T, c.N,
                       U, node_rows);
  } else {
    hipLaunchKernelGGL((sum_nodes_kernel<PB, OB, UPT, 256>), dim3(c.T),
                       dim3(256), 0, s, (const char *)part, node_slot,
                       (char *)out, c.T, c.N, U, node_rows);
  }
  return hipGetLastError();
}

}  // namespace

int node_rows_max(const moe_cfg &c) {
  return c.T * (c.K < c.N ? c.K : c.N);
}

hipError_t launch_pack_nodes(const moe_cfg &c, const void *x,
                             const int32_t *node_slot, void *node_send,
                             hipStream_t stream) {
  const int b = c.x_dtype == MOE_F32 ? 4 : 2;
  return launch_pack_rows(x, node_slot, c.N, node_rows_max(c), node_send,
                          c.T, c.H * b, stream);
}

hipError_t launch_forward(const moe_cfg &c, const void *node_send,
                          const int32_t *node_slot, const int32_t *topk_idx,
                          const int32_t *slot_pos, void *send,
                          hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int b = c.x_dtype == MOE_F32 ? 4 : 2;
  const int V = c.H * b / 16;
  const int need = (V + kWave - 1) / kWave;
  const int nr = node_rows_max(c);
  if (need <= 1) return launch_fwd<1>(c, node_send, node_slot, topk_idx, slot_pos, send, V, nr, stream);
  if (need <= 2) return launch_fwd<2>(c, node_send, node_slot, topk_idx, slot_pos, send, V, nr, stream);
  if (need <= 4) return launch_fwd<4>(c, node_send, node_slot, topk_idx, slot_pos, send, V, nr, stream);
  if (need <= 8) return launch_fwd<8>(c, node_send, node_slot, topk_idx, slot_pos, send, V, nr, stream);
  return launch_fwd<16>(c, node_send, node_slot, topk_idx, slot_pos, send, V, nr, stream);
}

hipError_t launch_partial(const moe_cfg &c, const void *y,
                          const int32_t *slot_pos, const float *topk_w,
                          const int32_t *topk_idx, const float *expert_scale,
                          const int32_t *node_slot, int part_dtype,
                          void *part, hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const bool yb = c.x_dtype == MOE_BF16, pb = part_dtype == MOE_BF16;
  const int nr = node_rows_max(c);
  if (yb && pb) return launch_partial_d<true, true>(c, y, slot_pos, topk_w, topk_idx, expert_scale, node_slot, part, nr, stream);
  if (yb && !pb) return launch_partial_d<true, false>(c, y, slot_pos, topk_w, topk_idx, expert_scale, node_slot, part, nr, stream);
  if (!yb && pb) return launch_partial_d<false, true>(c, y, slot_pos, topk_w, topk_idx, expert_scale, node_slot, part, nr, stream);
  return launch_partial_d<false, false>(c, y, slot_pos, topk_w, topk_idx, expert_scale, node_slot, part, nr, stream);
}

hipError_t launch_sum_nodes(const moe_cfg &c, const void *part, int part_dtype,
                            const int32_t *node_slot, void *out,
                            hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const bool pb = part_dtype == MOE_BF16, ob = c.out_dtype == MOE_BF16;
  const int nr = node_rows_max(c);
  if (pb && ob) return launch_sum_d<true, true>(c, part, node_slot, out, nr, stream);
  if (pb && !ob) return launch_sum_d<true, false>(c, part, node_slot, out, nr, stream);
  if (!pb && ob) return launch_sum_d<false, true>(c, part, node_slot, out, nr, stream);
  return launch_sum_d<false, false>(c, part, node_slot, out, nr, stream);
}

}  // namespace moe
