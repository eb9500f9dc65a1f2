// FP8 (E4M3) dispatch with per-block scales, and the combine of FP8 rows,
// for gfx950.
//
// "Efficient and portable mixture-of-experts communication", section
// "Envío (Dispatch)": tokens are sent with block scale factors; "Workload-
// Static Optical Circuit Switching for Scalable LLM Inference Decode",
// section "Communication precision": FP8 transport for MoE dispatch.  The
// format and block size are readings: OCP E4M3 codes (gfx950's native FP8
// conversions), one fp32 scale s = amax/448 per block of B elements, codes
// of fp32(x * fp32(448/amax)) clamped to +-448.  A packed row is H codes,
// then H/B scales, then zero padding to a multiple of 128 bytes, so rows
// start on 128-byte lines and no line holds parts of two rows.  Against a
// 16-byte stride (7392 against 7424 bytes for H = 7168, B = 128) the step
// of the DeepSeek-V3 shape took 480 instead of 503 us on MI355X: a row
// read or written no longer shares its first and last lines with the
// neighbouring rows, which other waves touch at other times.
//
// Pack: one wave per token.  A lane holds 8 consecutive elements of the row
// (one 16-byte bf16 vector); the B/8 lanes of a block reduce its amax with
// xor-shuffles, every lane converts its 8 elements with v_cvt_pk_fp8_f32 and
// the wave stores the codes (8 bytes a lane) and then the row's tail (block
// scales and padding, gathered in LDS) to the K destination rows.  The row
// is read once and quantised once per token.
//
// Combine: as the bf16 combine, with 16 codes (one 16-byte vector) and their
// block scale per unit; codes are widened with v_cvt_pk_f32_fp8 and
// accumulated as fmaf(w * s_e * scale, code, acc) in fp32.
#include <algorithm>

#include "moe_internal.h"
#include "row_io.h"

namespace moe {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// E4M3 codes of 4 fp32 values, packed little-endian in one word.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c,
                                           float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// L = B/8 lanes per block; VPL units of 8 elements per lane and pass.
// Codes go out as 8-byte stores, 512 contiguous bytes per instruction.  The
// row's tail (block scales, then zero padding up to the 128-byte row
// stride) is gathered in LDS, nd dwords per wave, and stored as whole
// dwords, so every line of a row is written in full by one wave.  Ordinary
// stores: with the 128-byte stride the pack took 212 us for the DeepSeek-V3
// shape against 248 us with device-scope non-temporal stores and 255 us with
// non-temporal ones (the combine after it then reads 25 us faster, which
// does not make up for it).
template <bool XB, int L, int VPL>
__global__ __launch_bounds__(256) void pack_fp8_kernel(
    const char *__restrict__ x, const int32_t *__restrict__ slot_pos,
    char *__restrict__ send, int T, int K, int U, int H, int rb, int rows) {
  extern __shared__ float tail_lds[];  // [4 waves][nd]
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const int t = blockIdx.x * (256 / kWave) + w;
  if (t >= T) return;  // one token per wave: uniform exit
  const int my_slot = lane < K ? slot_pos[(size_t)t * K + lane] : -1;
  const char *xrow = x + (size_t)t * U * (XB ? 16 : 32);
  const int nd = (rb - H) / 4;  // tail dwords: U / L scales, then padding
  float *tl = tail_lds + (size_t)w * nd;
  for (int q = U / L + lane; q < nd; q += kWave) tl[q] = 0.0f;

  for (int base = 0; base < U; base += kWave * VPL) {
    Unit<XB> u[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      u[j].load(xrow, min(base + j * kWave + lane, U - 1));
    u32x2 code[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(u[j].get(e)));
      // U is a multiple of L and every pass starts at a multiple of 64, so
      // the L lanes of a block are aligned; lanes past the row end form
      // whole blocks of their own and are never stored
#pragma unroll
      for (int off = 1; off < L; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
      const int i = base + j * kWave + lane;
      if (lane % L == 0 && i < U) tl[i / L] = a / 448.0f;
      const float r = 448.0f / a;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = u[j].get(e);
        // a block of zeros keeps its zeros (and their signs)
        p[e] = a == 0.0f ? v : fminf(fmaxf(v * r, -448.0f), 448.0f);
      }
      code[j][0] = e4m3x4(p[0], p[1], p[2], p[3]);
      code[j][1] = e4m3x4(p[4], p[5], p[6], p[7]);
    }
    for (int k = 0; k < K; ++k) {
      const int s = __builtin_amdgcn_readlane(my_slot, k);
      if ((unsigned)s >= (unsigned)rows) continue;  // out-of-range: skipped
      u32x2 *dst = (u32x2 *)(send + (size_t)s * rb);
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const int i = base + j * kWave + lane;
        if (i < U) dst[i] = code[j];
      }
    }
  }
  // the tail's LDS words were written by other lanes of this wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int k = 0; k < K; ++k) {
    const int s = __builtin_amdgcn_readlane(my_slot, k);
    if ((unsigned)s >= (unsigned)rows) continue;
    float *dst = (float *)(send + (size_t)s * rb + H);
    for (int q = lane; q < nd; q += kWave)
      dst[q] = tl[q];
  }
}

// 16 elements of a unit as fp32 from one 16-byte code vector.
__device__ __forceinline__ void deq16(const u32x4 &q, float *f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], true);
    f[4 * w + 0] = lo[0];
    f[4 * w + 1] = lo[1];
    f[4 * w + 2] = hi[0];
    f[4 * w + 3] = hi[1];
  }
}

// KT > 0: compile-time K; KT == 0: runtime K.  UPT units of 16 codes per
// thread and pass; L16 = B/16 units per block.  Row loads are branch-free
// (clamped to the last unit) as in the bf16 combine.
template <bool OB, int KT, int UPT, int TPT>
__global__ __launch_bounds__(256) void combine_fp8_kernel(
    const char *__restrict__ y, const int32_t *__restrict__ slot_pos,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ scale, char *__restrict__ out, int T, int Kr,
    int U16, int H, int L16, int rb, int rows) {
  const int K = KT > 0 ? KT : Kr;
  const int lane = threadIdx.x % kWave;
  const int tt = threadIdx.x % TPT;
  const int t = blockIdx.x * (256 / TPT) + threadIdx.x / TPT;
  if (t >= T) return;
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
  char *orow = out + (size_t)t * H * (OB ? 2 : 4);

  for (int base = 0; base < U16; base += TPT * UPT) {
    float acc[UPT][16];
#pragma unroll
    for (int j = 0; j < UPT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    if constexpr (KT > 0) {
      u32x4 q[KT][UPT];
      float bs[KT][UPT];
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const char *row =
            y + (size_t)__builtin_amdgcn_readlane(my_slot, k) * rb;
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
          const int i = min(base + j * TPT + tt, U16 - 1);
          q[k][j] = __builtin_nontemporal_load((const u32x4 *)row + i);
          bs[k][j] = *(const float *)(row + H + 4 * (i / L16));
        }
      }
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const float c = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(my_c), k));
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
          float f[16];
          deq16(q[k][j], f);
          const float cs = c * bs[k][j];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[j][e] = fmaf(cs, f[e], acc[j][e]);
        }
      }
    } else {
      for (int k = 0; k < K; ++k) {
        const char *row =
            y + (size_t)__builtin_amdgcn_readlane(my_slot, k) * rb;
        const float c = __int_as_float(
            __builtin_amdgcn_readlane(__float_as_int(my_c), k));
        u32x4 q[UPT];
        float bs[UPT];
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
          const int i = min(base + j * TPT + tt, U16 - 1);
          q[j] = __builtin_nontemporal_load((const u32x4 *)row + i);
          bs[j] = *(const float *)(row + H + 4 * (i / L16));
        }
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
          float f[16];
          deq16(q[j], f);
          const float cs = c * bs[j];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[j][e] = fmaf(cs, f[e], acc[j][e]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int i = base + j * TPT + tt;
      if (i < U16) {
        store_unit<OB>(orow, 2 * i, acc[j]);
        store_unit<OB>(orow, 2 * i + 1, acc[j] + 8);
      }
    }
  }
}

// Burst variant for large tables, as the bf16 combine's: persistent
// workgroups of one thread per 16-code unit (U16 <= 1024), G tokens at a
// time reduced (A at a time) into LDS staging laid out like out's rows,
// then written as one burst of non-temporal stores.  Measured on MI355X:
// 247 against 264 us for the DeepSeek-V3 shape, 871 against 882 us for the
// Kimi K2 shape; the FP8 rows are half the bytes of bf16 ones, so the
// output writes are a smaller share to gain on than in the bf16 combine.
// SV is the LDS staging in 16-byte vectors.  Below K = 16 it is 56 KiB, so
// two workgroups share a CU and one reduces while the other writes (247
// against 259 us with 112 KiB at K = 8); at K = 16 the 112 KiB stage of 8
// tokens is faster (871 against 898 us).
constexpr size_t kFp8BurstMinBytes = size_t(512) << 20;  // y rows

template <int KT>
constexpr int fp8_burst_vecs() {
  return KT >= 16 ? 7168 : 3584;
}

template <bool OB, int KT, int A, int SV>
__global__ __launch_bounds__(1024) void combine_fp8_burst_kernel(
    const char *__restrict__ y, const int32_t *__restrict__ slot_pos,
    const float *__restrict__ topk_w, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ scale, char *__restrict__ out, int T, int U16,
    int H, int L16, int rb, int G, int rows) {
  __shared__ u32x4 stage[SV];
  constexpr int kOV = OB ? 2 : 4;  // 16-byte output vectors per unit
  const int lane = threadIdx.x % kWave;
  const int u = threadIdx.x;
  const int uc = min(u, U16 - 1);
  const int ngroups = (T + G - 1) / G;
  for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
    const int t0 = g * G;
    const int nt = min(G, T - t0);
    for (int a = 0; a < nt; a += A) {  // A tokens' rows in flight together
      int my_slot[A];
      float my_c[A];
#pragma unroll
      for (int h = 0; h < A; ++h) {
        my_slot[h] = 0;
        my_c[h] = 0.0f;
        const int t = min(t0 + a + h, T - 1);
        if (lane < KT) {
          const size_t i = (size_t)t * KT + lane;
          my_slot[h] = slot_pos[i];
          my_c[h] = topk_w[i];
          if (scale) my_c[h] *= scale[topk_idx[i]];
          if ((unsigned)my_slot[h] >= (unsigned)rows) {  // out of range: 0
            my_slot[h] = 0;
            my_c[h] = 0.0f;
          }
        }
      }
      u32x4 q[A][KT];
      float bs[A][KT];
#pragma unroll
      for (int h = 0; h < A; ++h)
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          const char *row =
              y + (size_t)__builtin_amdgcn_readlane(my_slot[h], k) * rb;
          q[h][k] = __builtin_nontemporal_load((const u32x4 *)row + uc);
          bs[h][k] = *(const float *)(row + H + 4 * (uc / L16));
        }
#pragma unroll
      for (int h = 0; h < A; ++h) {
        float acc[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          const float c = __int_as_float(
              __builtin_amdgcn_readlane(__float_as_int(my_c[h]), k));
          float f[16];
          deq16(q[h][k], f);
          const float cs = c * bs[h][k];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = fmaf(cs, f[e], acc[e]);
        }
        if (u < U16 && a + h < nt) {
          u32x4 o[kOV];
          pack_unit<OB>(acc, o);
          pack_unit<OB>(acc + 8, o + kOV / 2);
#pragma unroll
          for (int j = 0; j < kOV; ++j)
            stage[((size_t)(a + h) * U16 + u) * kOV + j] = o[j];
        }
      }
    }
    __syncthreads();
    u32x4 *dst = (u32x4 *)out + (size_t)t0 * U16 * kOV;
    for (int i = threadIdx.x; i < nt * U16 * kOV; i += blockDim.x)
      __builtin_nontemporal_store(stage[i], dst + i);
    __syncthreads();
  }
}

template <bool XB, int L, int VPL>
hipError_t launch_pack_v(const moe_cfg &c, const void *x,
                         const int32_t *slot_pos, void *send, int rb,
                         hipStream_t s) {
  const int U = c.H / 8;
  const size_t lds = (size_t)4 * ((rb - c.H) / 4) * sizeof(float);
  hipLaunchKernelGGL((pack_fp8_kernel<XB, L, VPL>), dim3((c.T + 3) / 4),
                     dim3(256), lds, s, (const char *)x, slot_pos,
                     (char *)send, c.T, c.K, U, c.H, rb, c.T * c.K);
  return hipGetLastError();
}

template <bool XB, int L>
hipError_t launch_pack_l(const moe_cfg &c, const void *x,
                         const int32_t *slot_pos, void *send, int rb,
                         hipStream_t s) {
  const int need = (c.H / 8 + kWave - 1) / kWave;
  if (need <= 1) return launch_pack_v<XB, L, 1>(c, x, slot_pos, send, rb, s);
  if (need <= 2) return launch_pack_v<XB, L, 2>(c, x, slot_pos, send, rb, s);
  if (need <= 4) return launch_pack_v<XB, L, 4>(c, x, slot_pos, send, rb, s);
  if (need <= 8) return launch_pack_v<XB, L, 8>(c, x, slot_pos, send, rb, s);
  return launch_pack_v<XB, L, 16>(c, x, slot_pos, send, rb, s);
}

template <bool XB>
hipError_t launch_pack_b(const moe_cfg &c, int B, const void *x,
                         const int32_t *slot_pos, void *send, int rb,
                         hipStream_t s) {
  switch (B) {
    case 32: return launch_pack_l<XB, 4>(c, x, slot_pos, send, rb, s);
    case 64: return launch_pack_l<XB, 8>(c, x, slot_pos, send, rb, s);
    case 128: return launch_pack_l<XB, 16>(c, x, slot_pos, send, rb, s);
    default: return hipErrorInvalidValue;
  }
}

// Units per thread: about 16 code loads (plus their scales) per thread.
template <int KT>
constexpr int fp8_upt() {
  constexpr int kK = KT > 0 ? KT : 8;
  constexpr int raw = 16 / kK;
  return raw < 1 ? 1 : (raw > 8 ? 8 : raw);
}

template <bool OB, int KT>
hipError_t launch_comb_k(const moe_cfg &c, int B, const void *y,
                         const int32_t *slot_pos, const float *w,
                         const int32_t *idx, const float *scale, void *out,
                         int rb, hipStream_t s) {
  constexpr int UPT = fp8_upt<KT>();
  const int U16 = c.H / 16;
  if constexpr (KT > 0 && KT <= 16) {
    constexpr int kSV = fp8_burst_vecs<KT>();
    const int ov = OB ? 2 : 4;
    if (U16 <= 1024 && U16 * ov <= kSV &&
        (size_t)c.T * c.K * rb >= kFp8BurstMinBytes) {
      const int G = std::min(8, kSV / (U16 * ov));  // >= 1: one token fits
      const int ngroups = (c.T + G - 1) / G;
      constexpr int kA = KT >= 16 ? 1 : (16 / KT > 4 ? 4 : 16 / KT);  // rows in flight
      hipLaunchKernelGGL((combine_fp8_burst_kernel<OB, KT, kA, kSV>),
                         dim3(std::min(ngroups, 1024)),
                         dim3((U16 + kWave - 1) / kWave * kWave), 0, s,
                         (const char *)y, slot_pos, w, idx, scale, (char *)out,
                         c.T, U16, c.H, B / 16, rb, G, c.T * c.K);
      return hipGetLastError();
    }
  }
  if (U16 <= 64 * UPT) {
    hipLaunchKernelGGL((combine_fp8_kernel<OB, KT, UPT, 64>),
                       dim3((c.T + 3) / 4), dim3(256), 0, s, (const char *)y,
                       slot_pos, w, idx, scale, (char *)out, c.T, c.K, U16,
                       c.H, B / 16, rb, c.T * c.K);
  } else {
    hipLaunchKernelGGL((combine_fp8_kernel<OB, KT, UPT, 256>), dim3(c.T),
                       dim3(256), 0, s, (const char *)y, slot_pos, w, idx,
                       scale, (char *)out, c.T, c.K, U16, c.H, B / 16, rb,
                       c.T * c.K);
  }
  return hipGetLastError();
}

template <bool OB>
hipError_t launch_comb_d(const moe_cfg &c, int B, const void *y,
                         const int32_t *slot_pos, const float *w,
                         const int32_t *idx, const float *scale, void *out,
                         int rb, hipStream_t s) {
  switch (c.K) {
    case 1: return launch_comb_k<OB, 1>(c, B, y, slot_pos, w, idx, scale, out, rb, s);
    case 2: return launch_comb_k<OB, 2>(c, B, y, slot_pos, w, idx, scale, out, rb, s);
    case 4: return launch_comb_k<OB, 4>(c, B, y, slot_pos, w, idx, scale, out, rb, s);
    case 8: return launch_comb_k<OB, 8>(c, B, y, slot_pos, w, idx, scale, out, rb, s);
    case 16: return launch_comb_k<OB, 16>(c, B, y, slot_pos, w, idx, scale, out, rb, s);
    default: return launch_comb_k<OB, 0>(c, B, y, slot_pos, w, idx, scale, out, rb, s);
  }
}

}  // namespace

size_t fp8_row_bytes(int H, int B) {
  return ((size_t)H + 4 * (size_t)(H / B) + 127) & ~(size_t)127;
}

bool fp8_block_ok(const moe_cfg &c, int B) {
  if (!(B == 32 || B == 64 || B == 128) || c.H % B != 0 || c.H % 16 != 0)
    return false;
  // the pack keeps each of its 4 waves' row tail (H/B scales and up to 32
  // padding words) in LDS: at most 64 KiB a workgroup
  return (fp8_row_bytes(c.H, B) - (size_t)c.H) * 4 <= 65536;
}

hipError_t launch_pack_fp8(const moe_cfg &c, int B, const void *x,
                           const int32_t *slot_pos, void *send,
                           hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int rb = (int)fp8_row_bytes(c.H, B);
  return c.x_dtype == MOE_BF16
             ? launch_pack_b<true>(c, B, x, slot_pos, send, rb, stream)
             : launch_pack_b<false>(c, B, x, slot_pos, send, rb, stream);
}

hipError_t launch_combine_fp8(const moe_cfg &c, int B, const void *y,
                              const int32_t *slot_pos, const float *topk_w,
                              const int32_t *topk_idx,
                              const float *expert_scale, void *out,
                              hipStream_t stream) {
  if (c.T == 0) return hipSuccess;
  const int rb = (int)fp8_row_bytes(c.H, B);
  if (c.out_dtype == MOE_BF16)
    return launch_comb_d<true>(c, B, y, slot_pos, topk_w, topk_idx,
                               expert_scale, out, rb, stream);
  return launch_comb_d<false>(c, B, y, slot_pos, topk_w, topk_idx,
                              expert_scale, out, rb, stream);
}

}  // namespace moe
