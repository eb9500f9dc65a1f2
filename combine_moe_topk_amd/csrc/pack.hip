// Dispatch pack for gfx950: send[slot_pos[t,k]] = x[t], bit for bit.
//
// "Efficient and portable mixture-of-experts communication", section
// "Envío (Dispatch)": token rows are copied into contiguous chunks, one per
// destination, before they are sent; on one GPU the destination chunks are
// the expert-major segments of `send`.
//
// HBM-bound copy.  Main kernel: one wave per (token, piece of 128 16-byte
// vectors, pair of destinations), pairs fastest, so the W/2 waves that copy
// one piece of a row run side by side: the first one's load brings the
// piece into the cache and the others hit it, so x still crosses HBM about
// once.  Each wave loads its 2 KiB piece once and stores it to its two
// destination rows (wave-uniform: scalar loads of slots[t,k]); every load or
// store instruction moves 1 KiB contiguously, and stores are non-temporal
// with device scope (store_stream below): the rows of `send` are not read
// again by this kernel.
// Measured on MI355X with the combine running between packs (as in a real
// step): 358 us for the DeepSeek-V3 shape (K = 8) and 1505 us for the Kimi
// K2 shape (K = 16), against 388 and 1536 us for the kernel below, which
// reads a whole row once into registers and stores it W times with ordinary
// stores.  One destination per wave was as fast at K = 8 but 20% slower at
// K = 16; ordinary stores cost 17% at K = 8.  For destination tables of
// less than 1 GiB (Qwen3, Mixtral, decode shapes) the row kernel was the
// faster one (49 against 55 us at Qwen3's shape, 8.0 against 10.3 us for
// 128-token decode) and the combine after it ran faster too: its ordinary
// stores leave part of `send` in the 256 MB last-level cache.  So the piece
// kernel runs from 1 GiB of destination rows up (and below 2^31 waves of
// work), the row kernel otherwise.
// Both kernels serve any table of W <= 64 destination rows per token (K for
// the expert-major pack, N for the node-level pack); entries outside
// [0, rows) are skipped.
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

// Streaming store with device scope (sc1) as well as the non-temporal hint.
// Measured with the combine running between packs: 1402 against 1458 us for
// the Kimi K2 shape (K = 16) with the plain non-temporal store, and within
// noise for the DeepSeek-V3 shape (355 against 362 us); ordinary stores or
// scope bits without nt were slower (383-418 us), since the dirty lines they
// leave are written back during the next kernel.  The compiler has no
// builtin for these bits on a global store, hence the one-instruction asm
// (a store: nothing is read back into registers).
__device__ __forceinline__ void store_stream(u32x4 v, u32x4 *p) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(p), "v"(v)
               : "memory");
}

constexpr int kPieceVP = 2;  // 16-byte vectors per lane in a piece
constexpr int kPieceG = 2;   // destinations per wave
constexpr size_t kPieceMinBytes = size_t(1) << 30;  // destination rows

// Hardware workgroup b runs on XCD b % 8 (the dispatcher deals workgroups
// out to the XCDs in turn).  When a piece's NG destination groups span
// B = NG / 4 workgroups, the workgroups are renumbered in groups of 8 B so
// that the B sharing a piece of x run on one XCD and share its L2, rather
// than each of B XCDs fetching the piece from memory.  The last, partial
// group keeps its numbers.
__device__ __forceinline__ int piece_block(int b, int B, int nb) {
  const int span = 8 * B;
  if (B <= 1 || b >= nb - nb % span) return b;
  const int r = b % span;
  return b - r + B * (r % 8) + r / 8;
}

__global__ __launch_bounds__(256) void pack_piece_kernel(
    const u32x4 *__restrict__ x, const int32_t *__restrict__ slots,
    u32x4 *__restrict__ send, int W, int V, int P, int NG, int rows, int n) {
  const int lane = threadIdx.x % kWave;
  const int B = NG % 4 == 0 ? NG / 4 : 1;
  // wave index made wave-uniform so the index arithmetic runs on the SALU
  const int g = piece_block(blockIdx.x, B, gridDim.x) * (256 / kWave) +
                __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (g >= n) return;  // n = T*P*NG waves of work
  const int q = g % NG;  // NG = ceil(W / kPieceG) destination groups
  const int p = (g / NG) % P;
  const int t = g / (NG * P);
  const int base = p * kPieceVP * kWave + lane;
  const u32x4 *src = x + (size_t)t * V;
  u32x4 v[kPieceVP];  // clamped loads: no branch, all in flight together
#pragma unroll
  for (int j = 0; j < kPieceVP; ++j) v[j] = src[min(base + j * kWave, V - 1)];
#pragma unroll
  for (int d = 0; d < kPieceG; ++d) {
    const int k = q * kPieceG + d;
    if (k >= W) break;
    const int s = slots[(size_t)t * W + k];
    if ((unsigned)s >= (unsigned)rows) continue;  // out-of-range: skipped
    u32x4 *dst = send + (size_t)s * V;
#pragma unroll
    for (int j = 0; j < kPieceVP; ++j)
      if (base + j * kWave < V) store_stream(v[j], dst + base + j * kWave);
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
  const int P = (V + kWave * kPieceVP - 1) / (kWave * kPieceVP);
  const int NG = (W + kPieceG - 1) / kPieceG;
  const long n = (long)T * P * NG;
  if ((size_t)rows * row_bytes >= kPieceMinBytes && n <= 0x7fffffffL) {
    hipLaunchKernelGGL(pack_piece_kernel, dim3((unsigned)((n + 3) / 4)),
                       dim3(256), 0, stream, (const u32x4 *)x, slots,
                       (u32x4 *)dst, W, V, P, NG, rows, (int)n);
    return hipGetLastError();
  }
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
