// Dispatch pack for gfx950: send[slot_pos[t,k]] = x[t], bit for bit.
//
// "Efficient and portable mixture-of-experts communication", section
// "Envío (Dispatch)": token rows are copied into contiguous chunks, one per
// destination, before they are sent; on one GPU the destination chunks are
// the expert-major segments of `send`.
//
// HBM-bound copy: each x row is read once into registers (16-byte vectors,
// one wave per token, lanes striding the row so every load instruction moves
// 1 KiB contiguously) and stored K times with ordinary 16-byte stores.  The K
// destination rows are wave-uniform: lane k loads slot_pos[t,k] and the wave
// reads it back with readlane, so the store addresses come from SGPRs.  The
// same kernel serves any table of W <= 64 destination rows per token (K for
// the expert-major pack, N for the node-level pack); entries outside
// [0, rows) are skipped.
// Measured on MI355X with the combine running between packs (as in a real
// step): ordinary stores, which the last-level cache can merge before they
// reach HBM, beat non-temporal stores by ~11% (392 vs 441 us for the
// DeepSeek-V3 shape), and reach the chip's plain copy rate (~5.4 TB/s).
#include "moe_internal.h"

namespace moe {
namespace {

template <int VPL>
__global__ __launch_bounds__(256) void pack_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ slot_pos,
    u32x4 *__restrict__ send, int T, int W, int V, int rows) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // one token per wave: uniform exit
  const int my_slot = lane < W ? slot_pos[(size_t)t * W + lane] : -1;
  const u32x4 *src = x + (size_t)t * V;
  // blockIdx.y picks the part of the row when a row is split over waves
  const int chunk = (V + gridDim.y - 1) / gridDim.y;
  const int lo = blockIdx.y * chunk;
  const int hi = min(V, lo + chunk);
  for (int base = lo; base < hi; base += kWave * VPL) {
    u32x4 v[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int i = base + j * kWave + lane;
      if (i < hi) v[j] = src[i];
    }
    for (int k = 0; k < W; ++k) {
      const int s = __builtin_amdgcn_readlane(my_slot, k);
      if ((unsigned)s >= (unsigned)rows) continue;  // out-of-range: skipped
      u32x4 *dst = send + (size_t)s * V;
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int i = base + j * kWave + lane;
        if (i < hi) dst[i] = v[j];
      }
    }
  }
}

template <int VPL>
hipError_t launch_vpl(const void *x, const int32_t *slots, void *dst, int T,
                      int W, int V, int rows, int parts, hipStream_t s) {
  const dim3 grid((T + 3) / 4, parts);
  hipLaunchKernelGGL((pack_kernel<VPL>), grid, dim3(256), 0, s,
                     (const u32x4 *)x, slots, (u32x4 *)dst, T, W, V, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_rows(const void *x, const int32_t *slots, int W,
                            int rows, void *dst, int T, int row_bytes,
                            hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int V = row_bytes / 16;  // 16-byte vectors per row
  const int need = (V + kWave - 1) / kWave;
  // Few tokens (fewer than 2048 waves at one wave a token): one wave per
  // (token, 1 KiB piece of the row) instead, so the grid still fills the CUs.
  if (T < 2048 && need > 1)
    return launch_vpl<1>(x, slots, dst, T, W, V, rows, need, stream);
  if (need <= 1) return launch_vpl<1>(x, slots, dst, T, W, V, rows, 1, stream);
  if (need <= 2) return launch_vpl<2>(x, slots, dst, T, W, V, rows, 1, stream);
  if (need <= 4) return launch_vpl<4>(x, slots, dst, T, W, V, rows, 1, stream);
  if (need <= 8) return launch_vpl<8>(x, slots, dst, T, W, V, rows, 1, stream);
  return launch_vpl<16>(x, slots, dst, T, W, V, rows, 1, stream);
}

hipError_t launch_pack(const moe_cfg &c, const void *x,
                       const int32_t *slot_pos, void *send,
                       hipStream_t stream) {
  const int b = c.x_dtype == MOE_F32 ? 4 : 2;
  return launch_pack_rows(x, slot_pos, c.K, c.T * c.K, send, c.T, c.H * b,
                          stream);
}

}  // namespace moe
