// The fused step for decode-sized batches (a few hundred tokens): after the
// gate, one launch does the dispatch layout, the pack and the combine.
//
// What is computed is exactly the layout of "Efficient and portable
// mixture-of-experts communication", section "Envío (Dispatch)" (counts,
// exclusive offsets, the expert-major dispatch permutation), the node-level
// dedup of "Cobalt: Leveraging Expert Co-activation for Efficient
// Distributed MoE Training", Section 1, the pack send[slot_pos[t,k]] = x[t],
// and the combine of section "Combinación (Combine)", out[t] = sum_k
// w[t,k] s[e] send[slot_pos[t,k]] with fp32 fused multiply-adds in k order
// and one rounding: the same results, bit for bit, as the layout, pack and
// combine kernels.
//
// Why one launch.  At this size every step is a few microseconds of launch
// and dependent-latency chains over a few megabytes ("Workload-Static
// Optical Circuit Switching for Scalable LLM Inference Decode", section
// "Accelerators": small decode kernels reach a fraction of peak bandwidth
// and none takes under a few microseconds).  Two facts remove the grid-wide
// dependencies between the steps:
//   - a token's slots need only the expert ids of all tokens (T*K of them,
//     a few KB): every workgroup loads them and derives the counts and
//     offsets it needs with LDS histograms and a scan, instead of waiting
//     for a layout launch;
//   - the combine of token t reads exactly the K send rows that the pack of
//     token t wrote, so the workgroup that packs a token's rows combines
//     them: after a workgroup barrier its threads read the rows back from
//     send (never from x) and sum them.
// Workgroup 0 writes the batch-wide outputs (counts, offsets, node masks
// and node slots); workgroup 1 + t*P + p owns part p of token t's row, and
// parts p = 0 write the token's own layout outputs.
#include <algorithm>

#include "moe_internal.h"
#include "row_io.h"

namespace moe {
namespace {

constexpr int kDecodeMaxTokens = 1024;
constexpr int kDecodeMaxIds = 4096;       // T*K, held in registers
constexpr size_t kDecodeMaxLds = 65536;   // bytes of LDS a workgroup may use
constexpr int kDecodeBlock = 1024;
constexpr int kDecodeWaves = kDecodeBlock / kWave;

// Exclusive scan of n values in LDS by the whole workgroup into out[0..n]
// (out[n] = total).  Ends with a barrier.
__device__ void scan_lds(const int32_t *in, int n, int32_t *out,
                         int32_t *wsum) {
  const int B = blockDim.x;
  const int per = (n + B - 1) / B;
  const int lo = min(n, (int)threadIdx.x * per);
  const int hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += in[i];
  const int lane = threadIdx.x % kWave;
  int inc = local;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int v = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += v;
  }
  const int w = threadIdx.x / kWave;
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int v = 0; v < (B + kWave - 1) / kWave; ++v) {
      const int s = wsum[v];
      wsum[v] = run;
      run += s;
    }
    out[n] = run;
  }
  __syncthreads();
  int run = wsum[w] + inc - local;
  for (int i = lo; i < hi; ++i) {
    out[i] = run;
    run += in[i];
  }
  __syncthreads();
}

struct DecodeOut {
  int32_t *expert_count, *expert_off, *rank_count, *rank_off,
      *rank_token_count, *node_count, *node_off, *node_slot, *slot_pos,
      *row_src;
  uint64_t *node_mask;
};

// Inclusive sum over the lanes of a wave (DPP: row_shr:1,2,4,8 inside
// 16-lane rows, then row_bcast:15 into rows 1 and 3, row_bcast:31 into rows
// 2 and 3).
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = dpp_add<0x111, 0xF>(v);
  v = dpp_add<0x112, 0xF>(v);
  v = dpp_add<0x114, 0xF>(v);
  v = dpp_add<0x118, 0xF>(v);
  v = dpp_add<0x142, 0xA>(v);
  v = dpp_add<0x143, 0xC>(v);
  return v;
}

// The expert ids of the T*K slots a thread holds: slot i = tid + j*B
// (T*K <= 4096 over at least 256 threads: at most 16 a thread).
constexpr int kIdsPerThread = kDecodeMaxIds / 256;

struct Ids {
  int32_t e[kIdsPerThread];

  // ids written before this launch
  __device__ __forceinline__ void load(const int32_t *topk_idx, int TK) {
    const int B = blockDim.x, tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kIdsPerThread; ++j)
      if (j * B < TK) e[j] = tid + j * B < TK ? topk_idx[tid + j * B] : 0;
  }

};

// The batch-wide layout outputs, by workgroup 0: expert counts and offsets
// (an LDS histogram and a scan), and from per-node and per-rank bitmaps of
// the tokens (64 tokens a word, set with LDS atomics, the bitmaps of the
// layout kernels): distinct tokens per rank, node counts and offsets, and
// every token's node mask and node slots.
__device__ void decode_globals(const Ids &ids, int T, int E, int K, int R,
                               int N, uint32_t m_rank, uint32_t m_node,
                               uint32_t m_k, const DecodeOut &o,
                               uint64_t *sm) {
  const int tid = threadIdx.x, B = blockDim.x, lane = tid % kWave;
  const int TK = T * K;
  const int TW = (T + kWave - 1) / kWave;  // 64-token words of a bitmap
  uint64_t *nbm = sm;                      // [N][TW]
  uint64_t *rbm = nbm + (size_t)N * TW;    // [R][TW]
  int32_t *hist = (int32_t *)(rbm + (size_t)R * TW);  // [E]
  int32_t *eoff = hist + E;                // [E + 1]
  int32_t *pfx = eoff + E + 1;             // [N][TW] tokens before word w
  int32_t *noff = pfx + N * TW;            // [N + 1]
  int32_t *wsum = noff + N + 1;            // [kDecodeWaves]

  for (int i = tid; i < (N + R) * TW; i += B) nbm[i] = 0;  // nbm and rbm
  for (int i = tid; i < E; i += B) hist[i] = 0;
  __syncthreads();
  auto add = [&](int i, int e) {  // slot i = t*K + k with expert e
    if ((unsigned)e >= (unsigned)E) return;  // never produced by the gate
    atomicAdd(&hist[e], 1);
    const int j = div_small(i, m_k);
    const unsigned long long bit = 1ull << (j % kWave);
    const int w = j / kWave;
    atomicOr((unsigned long long *)&nbm[div_small(e, m_node) * TW + w], bit);
    atomicOr((unsigned long long *)&rbm[div_small(e, m_rank) * TW + w], bit);
  };
#pragma unroll
  for (int j = 0; j < kIdsPerThread; ++j)
    if (tid + j * B < TK) add(tid + j * B, ids.e[j]);
  __syncthreads();
  scan_lds(hist, E, eoff, wsum);  // ends with a barrier
  const int per_rank = E / R;
  for (int e = tid; e < E; e += B) {
    o.expert_count[e] = hist[e];
    o.expert_off[e] = eoff[e];
  }
  for (int r = tid; r < R; r += B) {
    o.rank_off[r] = eoff[r * per_rank];
    o.rank_count[r] = eoff[(r + 1) * per_rank] - eoff[r * per_rank];
    if (o.rank_token_count) {
      int c = 0;
      for (int w = 0; w < TW; ++w) c += __popcll(rbm[r * TW + w]);
      o.rank_token_count[r] = c;
    }
  }
  if (tid == 0) {
    o.expert_off[E] = eoff[E];
    o.rank_off[R] = eoff[E];
  }
  if (!o.node_mask && !o.node_slot && !o.node_count && !o.node_off) return;
  if (tid < N) {  // per node: tokens before each word, and the total
    int run = 0;
    for (int w = 0; w < TW; ++w) {
      pfx[tid * TW + w] = run;
      run += __popcll(nbm[tid * TW + w]);
    }
    noff[tid] = run;  // the count, for now
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int n = 0; n < N; ++n) {
      const int c = noff[n];
      if (o.node_count) o.node_count[n] = c;
      noff[n] = run;
      run += c;
    }
    noff[N] = run;
  }
  __syncthreads();
  if (o.node_off)
    for (int n = tid; n <= N; n += B) o.node_off[n] = noff[n];
  const uint64_t below = (1ull << lane) - 1;
  for (int j = tid; j < T; j += B) {
    const int w = j / kWave;
    uint64_t mask = 0;
    for (int n = 0; n < N; ++n) {
      const uint64_t word = nbm[n * TW + w];
      const bool has = (word >> (j % kWave)) & 1;
      mask |= (uint64_t)has << n;
      if (o.node_slot)
        o.node_slot[(size_t)j * N + n] =
            has ? noff[n] + pfx[n * TW + w] + __popcll(word & below) : -1;
    }
    if (o.node_mask) o.node_mask[j] = mask;
  }
}

template <bool YB, bool OB>
__global__ __launch_bounds__(kDecodeBlock) void decode_kernel(
    const char *__restrict__ x, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ topk_w, const float *__restrict__ scale,
    int T, int E, int K, int R, int N, int U, int P, uint32_t m_rank,
    uint32_t m_node, uint32_t m_k, DecodeOut o, char *__restrict__ send,
    char *__restrict__ out) {
  extern __shared__ uint64_t sm64[];
  const int TK = T * K;
  const int tid = threadIdx.x, B = blockDim.x;
  if (blockIdx.x == 0) {
    Ids ids;
    ids.load(topk_idx, TK);
    decode_globals(ids, T, E, K, R, N, m_rank, m_node, m_k, o, sm64);
    return;
  }
  int32_t *hist = (int32_t *)sm64;  // [E] slots per expert
  int32_t *hb = hist + E;           // [E] the same over the slots before t's
  int32_t *eoff = hb + E;           // [E] exclusive prefix of hist
  int32_t *slot = eoff + E;         // [32] token t's send rows
  float *coef = (float *)(slot + 32);  // [32] w * s of token t's slots

  const int b = blockIdx.x - 1;
  const int t = b / P;
  const int part = b % P;
  const int mine = t * K;

  // Every global load this workgroup needs is issued first, in the order
  // they are used (loads complete in issue order): the token's own expert
  // ids and gate weights, all expert ids, the token's row of x (on its way
  // while the slots are derived), then the token's expert scales.
  const int my_e = tid < K ? topk_idx[mine + tid] : 0;
  const float my_w = tid < K ? topk_w[mine + tid] : 0.0f;
  Ids ids;
  ids.load(topk_idx, TK);
  const int chunk = (U + P - 1) / P;
  const int u0 = part * chunk;
  const int u1 = min(U, u0 + chunk);
  constexpr int kVecs = YB ? 1 : 2;  // 16-byte vectors per 8-element unit
  const size_t rbytes = (size_t)U * 16 * kVecs;
  constexpr int kPre = 4;  // vectors of x a thread holds (more: reloaded)
  u32x4 xv[kPre];
  const u32x4 *xsrc = (const u32x4 *)(x + (size_t)t * rbytes);
#pragma unroll
  for (int q = 0; q < kPre; ++q)
    xv[q] = xsrc[min(u0 * kVecs + tid + q * B, U * kVecs - 1)];
  const bool my_ok = tid < K && (unsigned)my_e < (unsigned)E;
  const float sc = (my_ok && scale) ? scale[my_e] : 1.0f;

  // slot of (t, k) = slots of experts below e_k + slots of e_k before t's:
  // LDS histograms of every slot's expert and of the slots before t's (ids
  // outside [0, E), which the gate never produces, are left out), then one
  // wave's scan of the first
  for (int i = tid; i < 2 * E; i += B) hist[i] = 0;
  __syncthreads();
  auto count = [&](int i, int e) {
    if ((unsigned)e >= (unsigned)E) return;
    atomicAdd(&hist[e], 1);
    if (i < mine) atomicAdd(&hb[e], 1);
  };
#pragma unroll
  for (int j = 0; j < kIdsPerThread; ++j)
    if (tid + j * B < TK) count(tid + j * B, ids.e[j]);
  __syncthreads();
  if (tid < kWave) {
    const int per = (E + kWave - 1) / kWave;
    const int lo = min(E, tid * per), hi = min(E, lo + per);
    int local = 0;
    for (int e = lo; e < hi; ++e) local += hist[e];
    int run = wave_inclusive_scan(local) - local;
    for (int e = lo; e < hi; ++e) {
      eoff[e] = run;
      run += hist[e];
    }
  }
  __syncthreads();
  if (tid < K) {
    int s = -1;
    float c = 0.0f;
    if (my_ok) {
      s = eoff[my_e] + hb[my_e];
      c = scale ? my_w * sc : my_w;  // fp32 product, as the combine kernel
    }
    slot[tid] = s;
    coef[tid] = c;
    if (part == 0) {
      o.slot_pos[mine + tid] = s;
      if (s >= 0) o.row_src[s] = mine + tid;
    }
  }
  __syncthreads();

  // Pack: the token's row units, stored to each of its K send rows.  The
  // stores are non-temporal: the lines still serve the combine's reads
  // below from the cache, and fewer dirty lines are left to write back when
  // the kernel ends (7.7 against 8.1 us a launch for 128 tokens of the
  // DeepSeek-V3 shape; with the device-scope bit as well the reads below
  // missed the cache, 9.2 us).
  const int vend = u1 * kVecs;
#pragma unroll
  for (int q = 0; q < kPre; ++q) {
    const int v = u0 * kVecs + tid + q * B;
    if (v >= vend) break;
    for (int k = 0; k < K; ++k) {
      const int s = slot[k];
      if (s >= 0)
        __builtin_nontemporal_store(xv[q],
                                    (u32x4 *)(send + (size_t)s * rbytes) + v);
    }
  }
  for (int v = u0 * kVecs + tid + kPre * B; v < vend; v += B) {
    const u32x4 val = xsrc[v];
    for (int k = 0; k < K; ++k) {
      const int s = slot[k];
      if (s >= 0)
        __builtin_nontemporal_store(val,
                                    (u32x4 *)(send + (size_t)s * rbytes) + v);
    }
  }
  // The pack's stores are visible to every thread of the workgroup after
  // the barrier; the combine below reads them back from send.
  __syncthreads();

  char *orow = out + (size_t)t * U * (OB ? 16 : 32);
  for (int u = u0 + tid; u < u1; u += B) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 8) {
      Unit<YB> y[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {  // clamped, branch-free loads
        const int s = slot[min(k0 + q, K - 1)];
        y[q].load(send + (size_t)max(s, 0) * rbytes, u);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (k0 + q >= K || slot[k0 + q] < 0) continue;
        const float c = coef[k0 + q];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(c, y[q].get(e), acc[e]);
      }
    }
    store_unit<OB>(orow, u, acc);
  }
}

size_t decode_lds_bytes(const moe_cfg &c) {
  const size_t TW = (c.T + kWave - 1) / kWave;
  // workgroup 0: node and rank bitmaps, hist, eoff, pfx, noff, wsum
  const size_t g = 8 * (size_t)(c.N + c.R) * TW +
                   4 * ((size_t)c.E + c.E + 1 + TW * c.N + c.N + 1 +
                        kDecodeWaves);
  // token workgroups: hist, hb, eoff, then slot and coef (K <= 32)
  const size_t w = 4 * (3 * (size_t)c.E + 2 * 32);
  return std::max(g, w);
}

}  // namespace

bool decode_ok(const moe_cfg &c) {
  return c.T >= 1 && c.T <= kDecodeMaxTokens &&
         (long)c.T * c.K <= kDecodeMaxIds &&
         decode_lds_bytes(c) <= kDecodeMaxLds;
}

hipError_t launch_decode(const moe_cfg &c, const void *x,
                         const int32_t *topk_idx, const float *topk_w,
                         const float *expert_scale, const moe_layout &lay,
                         void *send, void *out, hipStream_t stream) {
  const int U = c.H / 8;
  // parts of a row per token: enough workgroups to reach every CU, with at
  // least 64 units (a wave's worth) in each part
  int P = 1;
  while (c.T * P < 256 && U / (P * 2) >= 64) P *= 2;
  const int B = std::min(kDecodeBlock,
                         std::max(256, ((U + P - 1) / P + kWave - 1) / kWave *
                                           kWave));
  DecodeOut o{lay.expert_count, lay.expert_off, lay.rank_count, lay.rank_off,
              lay.rank_token_count, lay.node_count, lay.node_off,
              lay.node_slot, lay.slot_pos, lay.row_src, lay.node_mask};
  const uint32_t m_rank = div_magic(c.E / c.R);
  const uint32_t m_node = div_magic(c.E / c.N);
  const uint32_t m_k = div_magic(c.K);  // slot index -> token
  const size_t lds = decode_lds_bytes(c);
  const dim3 grid(1 + c.T * P);  // workgroup 0: the batch-wide outputs
  const bool yb = c.x_dtype == MOE_BF16, ob = c.out_dtype == MOE_BF16;
#define MOE_DECODE(YB_, OB_)                                                \
  hipLaunchKernelGGL((decode_kernel<YB_, OB_>), grid, dim3(B), lds, stream, \
                     (const char *)x, topk_idx, topk_w, expert_scale, c.T,  \
                     c.E, c.K, c.R, c.N, U, P, m_rank, m_node, m_k, o,      \
                     (char *)send, (char *)out)
  if (yb && ob) MOE_DECODE(true, true);
  else if (yb) MOE_DECODE(true, false);
  else if (ob) MOE_DECODE(false, true);
  else MOE_DECODE(false, false);
#undef MOE_DECODE
  return hipGetLastError();
}

}  // namespace moe
