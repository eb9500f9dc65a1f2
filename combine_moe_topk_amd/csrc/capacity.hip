// Capacity-padded and bucketed dispatch layout for gfx950.
//
// "Workload-Static Optical Circuit Switching for Scalable LLM Inference
// Decode", section "Variable MoE Traffic and Regularization": every buffer
// between a source and a destination expert is padded to a fixed capacity
// so each step moves the same volume, and rows beyond the capacity are
// dropped; bucketing rounds each count up to one of q levels instead.
//
// Built on the dropless layout: its count and scan kernels give the
// per-expert counts and, per slot, the token-ascending rank inside the
// expert (dropless slot - dropless offset).  Then
//   cap_scan  (one workgroup): kept_e = min(count_e, Cmax), segment size
//             cap_e = smallest level >= kept_e, exclusive offsets, dropped
//   remap     (one thread per slot): slot = rank < Cmax ? off[e] + rank : -1
//             and row_src[slot] = t*K + k (row_src pre-filled with -1)
// Padding rows of the send buffer are zeroed by zero_rows_kernel.
#include "moe_internal.h"

namespace moe {
namespace {

struct Levels {
  int32_t v[kMaxLevels];
  int32_t q;
};

__global__ __launch_bounds__(1024) void cap_scan_kernel(
    const int32_t *__restrict__ count, int E, Levels lv,
    int32_t *__restrict__ cap, int32_t *__restrict__ off,
    int32_t *__restrict__ dropped) {
  __shared__ int32_t wsum[1024 / kWave];
  __shared__ int32_t wdrop[1024 / kWave];
  const int cmax = lv.v[lv.q - 1];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int carry = 0, drop_total = 0;
  for (int base = 0; base < E; base += blockDim.x) {
    const int e = base + threadIdx.x;
    int c = 0, d = 0;
    if (e < E) {
      const int n = count[e];
      const int kept = n < cmax ? n : cmax;
      d = n - kept;
      c = cmax;
      for (int j = lv.q - 1; j >= 0; --j)
        if (lv.v[j] >= kept) c = lv.v[j];
      cap[e] = c;
    }
    // inclusive scans of c and d across the workgroup
    int inc = c, dinc = d;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
      const int v = __shfl_up(inc, s, kWave);
      const int dv = __shfl_up(dinc, s, kWave);
      if (lane >= s) {
        inc += v;
        dinc += dv;
      }
    }
    if (lane == kWave - 1) {
      wsum[w] = inc;
      wdrop[w] = dinc;
    }
    __syncthreads();
    int before = carry, tot = 0, dtot = 0;
    for (int v = 0; v < (int)(blockDim.x / kWave); ++v) {
      if (v < w) before += wsum[v];
      tot += wsum[v];
      dtot += wdrop[v];
    }
    if (e < E) off[e] = before + inc - c;
    carry += tot;
    drop_total += dtot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    off[E] = carry;
    *dropped = drop_total;
  }
}

__global__ void remap_kernel(const int32_t *__restrict__ topk_idx,
                             const int32_t *__restrict__ dropless_off,
                             const int32_t *__restrict__ cap_off,
                             int32_t *__restrict__ slot_pos,
                             int32_t *__restrict__ row_src, int n, int E,
                             int cmax) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int e = topk_idx[i];
  if ((unsigned)e >= (unsigned)E) {
    slot_pos[i] = -1;
    return;
  }
  const int rank = slot_pos[i] - dropless_off[e];
  int s = -1;
  if (rank >= 0 && rank < cmax) {
    s = cap_off[e] + rank;
    row_src[s] = i;
  }
  slot_pos[i] = s;
}

// One wave per row: rows whose row_src is negative are set to zero.
__global__ __launch_bounds__(256) void zero_rows_kernel(
    const int32_t *__restrict__ row_src, u32x4 *__restrict__ rows, int n,
    int V) {
  const int lane = threadIdx.x % kWave;
  const int r = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (r >= n || row_src[r] >= 0) return;  // uniform per wave
  const u32x4 z = {0u, 0u, 0u, 0u};
  u32x4 *row = rows + (size_t)r * V;
  // non-temporal: ordinary stores leave up to 256 MB of dirty lines in the
  // last-level cache, written back while the next step's pack runs (its
  // time rose from ~360 to ~440 us for the DeepSeek-V3 shape)
  for (int i = lane; i < V; i += kWave) __builtin_nontemporal_store(z, row + i);
}

}  // namespace

bool levels_ok(const moe_cfg &c, const int32_t *levels, int q) {
  if (!levels || q < 1 || q > kMaxLevels) return false;
  for (int j = 0; j < q; ++j)
    if (levels[j] < 1 || (j > 0 && levels[j] <= levels[j - 1])) return false;
  return (int64_t)c.E * levels[q - 1] <= INT32_MAX;
}

size_t capacity_ws_bytes(const moe_cfg &c) {
  const LayoutGeom g = layout_geom(c);
  // dropless expert offsets (E+1), rank counts/offsets (2R+1), row_src (T*K)
  const size_t extra = ((size_t)(c.E + 1) + 2 * (size_t)c.R + 1 +
                        (size_t)c.T * c.K) * 4;
  return g.ws_bytes + ((extra + 255) & ~(size_t)255);
}

hipError_t launch_layout_capacity(const moe_cfg &c, const int32_t *topk_idx,
                                  const int32_t *levels, int q,
                                  const moe_capacity_layout &cl, void *ws,
                                  hipStream_t stream) {
  const LayoutGeom g = layout_geom(c);
  int32_t *tmp = (int32_t *)((char *)ws + g.ws_bytes);
  moe_layout dl{};
  dl.expert_count = cl.expert_count;
  dl.expert_off = tmp;                        // [E+1]
  dl.rank_count = tmp + c.E + 1;              // [R]
  dl.rank_off = dl.rank_count + c.R;          // [R+1]
  dl.row_src = dl.rank_off + c.R + 1;         // [T*K]
  dl.slot_pos = cl.slot_pos;                  // dropless slots, remapped below
  hipError_t e = launch_layout(c, topk_idx, dl, ws, stream);
  if (e != hipSuccess) return e;
  Levels lv{};
  for (int j = 0; j < q; ++j) lv.v[j] = levels[j];
  lv.q = q;
  hipLaunchKernelGGL(cap_scan_kernel, dim3(1), dim3(1024), 0, stream,
                     cl.expert_count, c.E, lv, cl.expert_cap, cl.expert_off,
                     cl.dropped);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int cmax = levels[q - 1];
  e = launch_fill_u32((uint32_t *)cl.row_src, 0xFFFFFFFFu,
                      (size_t)c.E * cmax, stream);
  if (e != hipSuccess) return e;
  const int n = c.T * c.K;
  if (n > 0) {
    hipLaunchKernelGGL(remap_kernel, dim3((n + 255) / 256), dim3(256), 0,
                       stream, topk_idx, dl.expert_off, cl.expert_off,
                       cl.slot_pos, cl.row_src, n, c.E, cmax);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_pack_capacity(const moe_cfg &c, const void *x,
                                const int32_t *slot_pos,
                                const int32_t *row_src, int n_rows,
                                void *send, hipStream_t stream) {
  const int b = c.x_dtype == MOE_F32 ? 4 : 2;
  hipError_t e = launch_pack_rows(x, slot_pos, c.K, n_rows, send, c.T,
                                  c.H * b, stream);
  if (e != hipSuccess || n_rows == 0) return e;
  const int V = c.H * b / 16;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((n_rows + 3) / 4), dim3(256), 0,
                     stream, row_src, (u32x4 *)send, n_rows, V);
  return hipGetLastError();
}

}  // namespace moe
