// Gate-weighted combine for gfx950:
//   out[t,:] = sum_k w[t,k] * s[e(t,k)] * y[slot_pos[t,k], :]
// accumulated in fp32 and rounded to nearest-even once into out's type.
//
// "Efficient and portable mixture-of-experts communication", section
// "Combinación (Combine)": the receiver reads each token's K expert rows and
// forms their weighted average into an externally allocated output; section
// "Fragmentación e paralelismo": the accumulation is fused into the gather.
//
// HBM-bound gather (K rows read per row written).  A token is owned by TPT
// threads (64 or 256); the threads stride the row in units of 8 elements, so
// each load instruction of the group reads TPT*16 contiguous bytes of one
// expert row.  Lane k < K of every wave loads (slot, weight*scale) of slot k
// and the wave broadcasts them with readlane, so row addresses are scalar.
// Each thread owns UPT units of the row and issues all K*UPT of its 16-byte
// row loads back to back before the first FMA: UPT is the largest value that
// keeps about 32 loads (128 VGPRs of payload) in flight per thread, and TPT
// the narrowest group for which TPT*UPT units cover the row, so a token takes
// one pass when it fits.  Row loads are non-temporal (each y row is read
// exactly once), and so are the output stores.  Measured on MI355X for the
// DeepSeek-V3 shape (H=7168, K=8), with a pack before every combine as in a
// real step: one pass of 32 loads per thread takes ~385 us against ~425 us
// for two passes of 16, and non-temporal loads and stores beat ordinary ones
// by ~20% and ~9%; the L2 scope bits (sc0/sc1) change nothing.
#include <algorithm>

#include "moe_internal.h"
#include "row_io.h"

namespace moe {
namespace {

// KT > 0: K known at compile time (fully unrolled); KT == 0: runtime K.
// TPT: threads per token (64 or 256); UPT: 8-element units per thread and pass.
// Row loads are branch-free: a unit index past the row end is clamped to the
// row's last unit (an in-bounds address) and its value is never stored.  A
// guarded load would sit in its own basic block, and the compiler then waits
// for all outstanding loads before each one, serialising the K*UPT loads.
template <bool YBF16, bool OBF16, int KT, int UPT, int TPT>
__global__ __launch_bounds__(256) void combine_kernel(
    const char *__restrict__ y, const int32_t *__restrict__ slot_pos,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ scale, char *__restrict__ out, int T, int Kr,
    int U, int rows) {
  const int K = KT > 0 ? KT : Kr;
  const int lane = threadIdx.x % kWave;
  const int tt = threadIdx.x % TPT;  // thread within the token's group
  const int t = blockIdx.x * (256 / TPT) + threadIdx.x / TPT;
  if (t >= T) return;  // whole waves leave together (TPT is a wave multiple)
  const size_t ybytes = (size_t)U * (YBF16 ? 16 : 32);
  const size_t obytes = (size_t)U * (OBF16 ? 16 : 32);

  int my_slot = 0;
  float my_c = 0.0f;
  if (lane < K) {
    const size_t i = (size_t)t * K + lane;
    my_slot = slot_pos[i];
    my_c = topk_w[i];
    if (scale) my_c *= scale[topk_idx[i]];
    if ((unsigned)my_slot >= (unsigned)rows) {  // out of range: adds 0
      my_slot = 0;
      my_c = 0.0f;
    }
  }
  char *orow = out + (size_t)t * obytes;
  // blockIdx.y picks the part of the row when a row is split over blocks
  const int chunk = (U + gridDim.y - 1) / gridDim.y;
  const int lo = blockIdx.y * chunk;
  const int hi = min(U, lo + chunk);

  for (int base = lo; base < hi; base += TPT * UPT) {
    float acc[UPT][8];
#pragma unroll
    for (int j = 0; j < UPT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] = 0.0f;

    if constexpr (KT > 0) {
      Unit<YBF16> u[KT][UPT];
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const int s = __builtin_amdgcn_readlane(my_slot, k);
        const char *row = y + (size_t)s * ybytes;
#pragma unroll
        for (int j = 0; j < UPT; ++j)
          u[k][j].load(row, min(base + j * TPT + tt, hi - 1));
      }
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const float c = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(my_c), k));
#pragma unroll
        for (int j = 0; j < UPT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[j][e] = fmaf(c, u[k][j].get(e), acc[j][e]);
      }
    } else {
      for (int k = 0; k < K; ++k) {
        const int s = __builtin_amdgcn_readlane(my_slot, k);
        const float c = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(my_c), k));
        const char *row = y + (size_t)s * ybytes;
        Unit<YBF16> u[UPT];
#pragma unroll
        for (int j = 0; j < UPT; ++j)
          u[j].load(row, min(base + j * TPT + tt, hi - 1));
#pragma unroll
        for (int j = 0; j < UPT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            acc[j][e] = fmaf(c, u[j].get(e), acc[j][e]);
      }
    }
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int i = base + j * TPT + tt;
      if (i < hi) store_unit<OBF16>(orow, i, acc[j]);
    }
  }
}

constexpr size_t kBurstMinBytes = size_t(1) << 30;  // y rows
constexpr int kBurstBlocks = 1024;                    // persistent grid

// Burst variant, for tables of y rows of 1 GiB or more.  Persistent
// workgroups of one thread per 8-element unit (U <= 1024 units); a workgroup
// takes G consecutive tokens at a time, reduces them A at a time (A*K row
// loads in flight per thread) into LDS staging laid out like out's rows,
// then writes the G rows, which are contiguous in out, as one burst of
// non-temporal stores.  Measured on MI355X with a pack before every combine:
// 348 against 368 us for the DeepSeek-V3 shape and 1324 against 1470 us for
// the Kimi K2 shape (K = 16); output writes spread through the reads cost
// more than the same writes gathered into bursts.  For tables that fit the
// 256 MB last-level cache (Qwen3, Mixtral) the kernel above was as fast or
// faster (54 vs 59 us for Qwen3).
constexpr int kBurstVecs = 7168;  // 112 KiB of LDS staging per workgroup

template <bool YBF16, bool OBF16, int KT, int A>
__global__ __launch_bounds__(1024) void combine_burst_kernel(
    const char *__restrict__ y, const int32_t *__restrict__ slot_pos,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ scale, char *__restrict__ out, int T, int U,
    int G, int rows) {
  __shared__ u32x4 stage[kBurstVecs];
  constexpr int kOV = OBF16 ? 1 : 2;  // 16-byte vectors per output unit
  const int lane = threadIdx.x % kWave;
  const int u = threadIdx.x;  // this thread's unit of every row
  const int uc = min(u, U - 1);
  const size_t ybytes = (size_t)U * (YBF16 ? 16 : 32);
  const int ngroups = (T + G - 1) / G;
  for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int t0 = g * G;
    const int nt = min(G, T - t0);  // tokens in this group
    for (int a = 0; a < nt; a += A) {
      int my_slot[A];
      float my_c[A];
#pragma unroll
      for (int h = 0; h < A; ++h) {  // lane k < K: routing of token a+h
        my_slot[h] = 0;
        my_c[h] = 0.0f;
        const int t = min(t0 + a + h, T - 1);
        if (lane < KT) {
          const size_t i = (size_t)t * KT + lane;
          my_slot[h] = slot_pos[i];
          my_c[h] = topk_w[i];
          if (scale) my_c[h] *= scale[topk_idx[i]];
          if ((unsigned)my_slot[h] >= (unsigned)rows) {  // out of range: adds 0
            my_slot[h] = 0;
            my_c[h] = 0.0f;
          }
        }
      }
      Unit<YBF16> v[A][KT];
#pragma unroll
      for (int h = 0; h < A; ++h)
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          const int s = __builtin_amdgcn_readlane(my_slot[h], k);
          v[h][k].load(y + (size_t)s * ybytes, uc);
        }
#pragma unroll
      for (int h = 0; h < A; ++h) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          const float c = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(my_c[h]), k));
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(c, v[h][k].get(e), acc[e]);
        }
        if (u < U && a + h < nt) {
          u32x4 o[kOV];
          pack_unit<OBF16>(acc, o);
#pragma unroll
          for (int q = 0; q < kOV; ++q)
            stage[((size_t)(a + h) * U + u) * kOV + q] = o[q];
        }
      }
    }
    __syncthreads();
    u32x4 *dst = (u32x4 *)out + (size_t)t0 * U * kOV;
    for (int i = threadIdx.x; i < nt * U * kOV; i += blockDim.x)
      __builtin_nontemporal_store(stage[i], dst + i);
    __syncthreads();
  }
}

// Units per thread: about 32 16-byte row loads in flight per thread.
template <bool YB, int KT>
constexpr int upt_for() {
  constexpr int kLoadsPerUnit = YB ? 1 : 2;
  constexpr int kK = KT > 0 ? KT : 8;
  constexpr int raw = 32 / (kK * kLoadsPerUnit);
  return raw < 1 ? 1 : (raw > 8 ? 8 : raw);
}

template <bool YB, bool OB, int KT, int TPT, int UPT = upt_for<YB, KT>()>
hipError_t launch_kt(const moe_cfg &c, const void *y, const int32_t *slot_pos,
                     const float *w, const int32_t *idx, const float *scale,
                     void *out, int rows, int parts, hipStream_t s) {
  constexpr int kTokensPerBlock = 256 / TPT;
  const int U = c.H / 8;
  const dim3 grid((c.T + kTokensPerBlock - 1) / kTokensPerBlock, parts);
  hipLaunchKernelGGL((combine_kernel<YB, OB, KT, UPT, TPT>), grid, dim3(256),
                     0, s, (const char *)y, slot_pos, w, idx, scale,
                     (char *)out, c.T, c.K, U, rows);
  return hipGetLastError();
}

// The burst kernel's fixed choices for one (dtypes, K): tokens reduced at
// a time (about 8 row loads in flight per thread, at most 64 VGPRs of row
// payload), and whether it applies at all.
template <bool YB, int KT>
constexpr int burst_a() {
  constexpr int kLoads = (KT > 0 ? KT : 8) * (YB ? 1 : 2);  // KT 0: unused
  return kLoads >= 8 ? 1 : 8 / kLoads;
}

template <bool YB, bool OB, int KT>
hipError_t launch_k(const moe_cfg &c, const void *y, const int32_t *slot_pos,
                    const float *w, const int32_t *idx, const float *scale,
                    void *out, int rows, hipStream_t s) {
  const int U = c.H / 8;
  constexpr int kA = burst_a<YB, KT>();
  constexpr bool kBurstOk = KT > 0 && kA * KT * (YB ? 4 : 8) <= 64;
  if constexpr (kBurstOk) {
    const size_t ybytes = (size_t)U * (YB ? 16 : 32);
    if (U <= 1024 && (size_t)rows * ybytes >= kBurstMinBytes) {
      const int ov = OB ? 1 : 2;
      const int G = std::min(8, kBurstVecs / (U * ov));  // tokens per burst
      const int ngroups = (c.T + G - 1) / G;
      const int threads = (U + kWave - 1) / kWave * kWave;
      hipLaunchKernelGGL((combine_burst_kernel<YB, OB, KT, kA>),
                         dim3(std::min(ngroups, kBurstBlocks)), dim3(threads),
                         0, s, (const char *)y, slot_pos, w, idx, scale,
                         (char *)out, c.T, U, G, rows);
      return hipGetLastError();
    }
  }
  // Few tokens: one unit per thread, a wave per token and the row split in
  // 64-unit parts over blockIdx.y, so the grid still fills the CUs.
  if (c.T < 1024 && U > 64)
    return launch_kt<YB, OB, KT, 64, 1>(c, y, slot_pos, w, idx, scale, out,
                                        rows, (U + 63) / 64, s);
  // one wave per token while 64*UPT units cover the row, else a workgroup
  if (U <= 64 * upt_for<YB, KT>())
    return launch_kt<YB, OB, KT, 64>(c, y, slot_pos, w, idx, scale, out, rows, 1, s);
  return launch_kt<YB, OB, KT, 256>(c, y, slot_pos, w, idx, scale, out, rows, 1, s);
}

template <bool YB, bool OB>
hipError_t launch_d(const moe_cfg &c, const void *y, const int32_t *slot_pos,
                    const float *w, const int32_t *idx, const float *scale,
                    void *out, int rows, hipStream_t s) {
  switch (c.K) {
    case 1: return launch_k<YB, OB, 1>(c, y, slot_pos, w, idx, scale, out, rows, s);
    case 2: return launch_k<YB, OB, 2>(c, y, slot_pos, w, idx, scale, out, rows, s);
    case 4: return launch_k<YB, OB, 4>(c, y, slot_pos, w, idx, scale, out, rows, s);
    case 8: return launch_k<YB, OB, 8>(c, y, slot_pos, w, idx, scale, out, rows, s);
    case 16: return launch_k<YB, OB, 16>(c, y, slot_pos, w, idx, scale, out, rows, s);
    default: return launch_k<YB, OB, 0>(c, y, slot_pos, w, idx, scale, out, rows, s);
  }
}

}  // namespace

hipError_t launch_combine(const moe_cfg &c, const void *y,
                          const int32_t *slot_pos, const float *topk_w,
                          const int32_t *topk_idx, const float *expert_scale,
                          void *out, hipStream_t stream, int rows) {
  if (c.T == 0) return hipSuccess;
  if (rows < 0) rows = c.T * c.K;
  const bool yb = c.x_dtype == MOE_BF16;
  const bool ob = c.out_dtype == MOE_BF16;
  if (yb && ob)
    return launch_d<true, true>(c, y, slot_pos, topk_w, topk_idx, expert_scale, out, rows, stream);
  if (yb && !ob)
    return launch_d<true, false>(c, y, slot_pos, topk_w, topk_idx, expert_scale, out, rows, stream);
  if (!yb && ob)
    return launch_d<false, true>(c, y, slot_pos, topk_w, topk_idx, expert_scale, out, rows, stream);
  return launch_d<false, false>(c, y, slot_pos, topk_w, topk_idx, expert_scale, out, rows, stream);
}

}  // namespace moe
