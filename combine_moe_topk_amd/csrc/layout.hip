// Dispatch layout for gfx950: counts, exclusive offsets, node-level dedup and
// the stable expert-major dispatch permutation, with no atomics whose order
// could change a result.
//
// What is computed follows "Efficient and portable mixture-of-experts
// communication", section "Envío (Dispatch)" (the sender counts the tokens
// bound for every destination expert; the receiver packs them into contiguous
// per-expert buffers and records where each row came from), "Workload-Static
// Optical Circuit Switching for Scalable LLM Inference Decode", section
// "Variable MoE Traffic and Regularization" (rows per destination group), and
// "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
// Training", Section 1 (a token crosses to a node once, however many of its
// experts live there).
//
// Design.  A workgroup owns a tile of 64*W consecutive tokens, one token per
// lane.  For every wave and every expert (and rank, and node) it keeps a
// 64-bit LDS bitmap of the wave's tokens that select it, built with LDS
// atomicOr (order-free).  Then
//   count of expert e in the tile          = sum over waves of popcount
//   rank of (t, e) among earlier tile rows = popcount(bitmap & lanes-below)
//                                            + popcounts of earlier waves
// which is exactly the token-ascending order inside each expert, with no
// sorting and no order-dependent atomics.  When all tokens fit in one tile,
// one workgroup does everything (layout_block_kernel).  Otherwise three
// launches:
//   count: per-tile column counts (experts | ranks | nodes) + node masks
//   scan : the count table to per-tile exclusive prefixes and column totals
//          (one workgroup up to 32 tiles, which also writes the offsets;
//          else column-parallel, and the rank workgroups derive the
//          offsets from the totals); none for a small table (up to 64
//          tiles of 64 columns), whose raw counts every rank workgroup
//          sums itself
//   rank : rebuilds the tile bitmaps and writes slot_pos, row_src, node_slot
// In the fused call the gate can write the counts itself (gate.hip), and
// only scan and rank run here.  The count table lives in the caller's
// workspace: (nblocks + 1) x (E + R + N), the last row for the totals.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void raise_error(int32_t *err, int bits) {
  if (bits) atomicOr(err, bits);
}

// A token's K expert ids into registers, KM >= K of them: the index of every
// load is clamped into the row, so the loads have no branches and all go out
// before the first use (a guarded or data-dependent loop would wait for
// each load in turn: K memory round trips instead of one).
template <int KM>
__device__ __forceinline__ void load_ids(const int32_t *row, int K,
                                         int (&ev)[KM]) {
#pragma unroll
  for (int k = 0; k < KM; ++k) ev[k] = row[min(k, K - 1)];
}

template <int KM>
__global__ __launch_bounds__(1024) void layout_count_kernel(
    const int32_t *__restrict__ idx, int T, int K, int E, int R, int N,
    uint32_t m_rank, uint32_t m_node, uint64_t *__restrict__ node_mask,
    int32_t *__restrict__ table, int32_t *__restrict__ err) {
  extern __shared__ uint64_t bm[];  // [W][cols]
  const int cols = E + R + N;
  const int W = blockDim.x / kWave;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  int ev[KM];
  if (t < T) load_ids<KM>(idx + (size_t)t * K, K, ev);
  for (int i = threadIdx.x; i < W * cols; i += blockDim.x) bm[i] = 0;
  __syncthreads();

  const uint64_t bit = 1ull << lane;
  uint64_t *mine = bm + (size_t)w * cols;
  int bad = 0;
  if (t < T) {
    uint64_t mask = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k >= K) break;
      const int e = ev[k];
      if ((unsigned)e >= (unsigned)E) {
        bad |= MOE_DEVERR_EXPERT_RANGE;
        continue;
      }
      const uint64_t old = atomicOr((unsigned long long *)&mine[e], bit);
      if (old & bit) bad |= MOE_DEVERR_DUP_EXPERT;
      atomicOr((unsigned long long *)&mine[E + div_small(e, m_rank)], bit);
      mask |= 1ull << div_small(e, m_node);
    }
    for (uint64_t m = mask; m; m &= m - 1)
      atomicOr((unsigned long long *)&mine[E + R + __ffsll((long long)m) - 1],
               bit);
    if (node_mask) node_mask[t] = mask;
  }
  raise_error(err, bad);
  __syncthreads();

  int32_t *out = table + (size_t)blockIdx.x * cols;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) {
    int s = 0;
    for (int v = 0; v < W; ++v) s += __popcll(bm[(size_t)v * cols + c]);
    out[c] = s;
  }
}

// Exclusive scan of n <= 4096 LDS values by one 1024-thread workgroup.
// Writes out[0..n] (out[n] = total) to LDS.
__device__ void block_exclusive_scan(const int32_t *in, int n, int32_t *out) {
  __shared__ int32_t wsum[1024 / kWave];
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int lo = min(n, (int)threadIdx.x * per);
  const int hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += in[i];
  // inclusive scan of `local` across the wave
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
    for (int v = 0; v < (int)(blockDim.x / kWave); ++v) {
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

__global__ __launch_bounds__(1024) void layout_scan_kernel(
    int32_t *__restrict__ table, int nblocks, int E, int R, int N,
    int per_rank, int32_t *__restrict__ expert_count,
    int32_t *__restrict__ expert_off, int32_t *__restrict__ rank_count,
    int32_t *__restrict__ rank_off, int32_t *__restrict__ rank_token_count,
    int32_t *__restrict__ node_count, int32_t *__restrict__ node_off) {
  extern __shared__ int32_t sm32[];
  const int cols = E + R + N;
  int32_t *tot = sm32;              // [cols]
  int32_t *eoff = sm32 + cols;      // [E + 1]
  // Column-wise exclusive prefix over the tiles, in place.  A thread owns
  // a column and takes its rows 16 at a time: the 16 loads are issued
  // before any store (stores to the table would otherwise order every later
  // load behind them), so a chunk costs one memory round trip.  (Chunks of
  // 64 were slower: 9.8 against 6.9 us for 64 tiles; so were 64 or 32 rows
  // a chunk with unconditional clamped loads, 1 or 2 columns a thread; two
  // chunk buffers used in turn, each chunk's loads issued before the
  // previous chunk's stores, changed nothing: 23.2 against 22.6 us for the
  // whole DeepSeek-V3 layout, 45.4 against 45.6 us for Kimi K2.)
  constexpr int kChunk = 16;
  for (int c = threadIdx.x; c < cols; c += blockDim.x) {
    int run = 0;
    for (int b0 = 0; b0 < nblocks; b0 += kChunk) {
      int32_t *p = table + (size_t)b0 * cols + c;
      const int n = min(kChunk, nblocks - b0);
      int v[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) v[j] = j < n ? p[(size_t)j * cols] : 0;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (j < n) p[(size_t)j * cols] = run;
        run += v[j];
      }
    }
    tot[c] = run;
  }
  __syncthreads();
  block_exclusive_scan(tot, E, eoff);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    expert_count[e] = tot[e];
    expert_off[e] = eoff[e];
  }
  if (threadIdx.x == 0) expert_off[E] = eoff[E];
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    rank_off[r] = eoff[r * per_rank];
    rank_count[r] = eoff[(r + 1) * per_rank] - eoff[r * per_rank];
    if (rank_token_count) rank_token_count[r] = tot[E + r];
  }
  if (threadIdx.x == 0) rank_off[R] = eoff[E];
  // Tail row (index nblocks): global exclusive offsets of the expert and
  // node columns, read by the rank kernel.
  int32_t *tail = table + (size_t)nblocks * cols;
  for (int e = threadIdx.x; e < E; e += blockDim.x) tail[e] = eoff[e];
  if (threadIdx.x == 0) {
    int run = 0;
    for (int n = 0; n < N; ++n) {
      const int v = tot[E + R + n];
      if (node_count) node_count[n] = v;
      if (node_off) node_off[n] = run;
      tail[E + R + n] = run;
      run += v;
    }
    if (node_off) node_off[N] = run;
  }
}

// Column-parallel scan of the count table, many workgroups: workgroup b
// takes 64 columns, and each column's tile rows are split into 16 chunks,
// one thread a chunk.  A thread sums its chunk, the chunk sums are scanned
// in LDS, and the thread writes the exclusive prefixes of its chunk in
// place; the tail row (index nblocks) gets each column's total.  Loads go
// out 8 at a time with clamped indexes (the empty asm keeps every loaded
// value used, so no load waits alone in a branch).
constexpr int kScanCols = 64;
constexpr int kScanChunks = 16;
// Up to this many tiles one workgroup scans the whole table (measured on
// MI355X: with 16 tiles, the Mixtral shape, its scan and rank launches
// took 8.1 us against 9.1 us for the column-parallel pair; with 64 tiles,
// the DeepSeek-V3 shape, 16.3 against 15.6 us, and with 128, Kimi K2's,
// 36.2 against 23.4 us).
constexpr int kSmallTable = 32;

__global__ __launch_bounds__(1024) void layout_scan_cols_kernel(
    int32_t *__restrict__ table, int nblocks, int cols) {
  __shared__ int32_t part[kScanChunks][kScanCols];
  const int cl = threadIdx.x % kScanCols;
  const int ch = threadIdx.x / kScanCols;
  const int c0 = (int)blockIdx.x * kScanCols + cl;
  const int c = min(c0, cols - 1);
  const bool col_ok = c0 < cols;
  const int per = (nblocks + kScanChunks - 1) / kScanChunks;
  const int r0 = min(nblocks, ch * per);
  const int r1 = min(nblocks, r0 + per);
  int32_t *col = table + c;
  // the chunk's first 8 rows stay in registers for the prefix pass (up to
  // 128 tiles that is the whole chunk); later rows are loaded again
  int v0[8];
  int sum = 0;
  for (int r = r0; r < r1; r += 8) {
    int v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = col[(size_t)min(r + q, r1 - 1) * cols];
#pragma unroll
    for (int q = 0; q < 8; ++q) asm volatile("" : "+v"(v[q]));
#pragma unroll
    for (int q = 0; q < 8; ++q) sum += r + q < r1 ? v[q] : 0;
    if (r == r0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v0[q] = v[q];
    }
  }
  part[ch][cl] = sum;
  __syncthreads();
  int run = 0;
  for (int q = 0; q < ch; ++q) run += part[q][cl];
  if (!col_ok) return;
  if (ch == kScanChunks - 1) col[(size_t)nblocks * cols] = run + sum;
  for (int r = r0; r < r1; r += 8) {
    int v[8];
    if (r == r0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = v0[q];
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = col[(size_t)min(r + q, r1 - 1) * cols];
#pragma unroll
      for (int q = 0; q < 8; ++q) asm volatile("" : "+v"(v[q]));
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (r + q < r1) {
        col[(size_t)(r + q) * cols] = run;
        run += v[q];
      }
    }
  }
}

// Inclusive scan over the 64 lanes of a wave with DPP: shifts by 1, 2, 4
// and 8 lanes inside each 16-lane row (a lane with no source adds 0), then
// the last lane of row 0 added into rows 1 and 3 (row_bcast:15) and the last
// lane of row 1 into rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROWS, int BANKS>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, BANKS, false);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = dpp_add<0x111, 0xF, 0xF>(v);  // row_shr:1
  v = dpp_add<0x112, 0xF, 0xF>(v);  // row_shr:2
  v = dpp_add<0x114, 0xF, 0xF>(v);  // row_shr:4
  v = dpp_add<0x118, 0xF, 0xF>(v);  // row_shr:8
  v = dpp_add<0x142, 0xA, 0xF>(v);  // row_bcast:15 into rows 1, 3
  v = dpp_add<0x143, 0xC, 0xF>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// Exclusive scan of a[0..n) in LDS, in place, by the whole workgroup
// (blockDim a multiple of 64, at most 1024); a[n] gets the total.  Ends
// with a barrier.
__device__ void scan_inplace(int32_t *a, int n, int32_t *wsum) {
  const int B = blockDim.x;
  const int per = (n + B - 1) / B;
  const int lo = min(n, (int)threadIdx.x * per);
  const int hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += a[i];
  const int lane = threadIdx.x % kWave;
  const int inc = wave_inclusive_scan(local);
  const int w = threadIdx.x / kWave;
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  if (w == 0) {  // wave 0 scans the wave sums (at most 16)
    const int nw = B / kWave;
    const int s = lane < nw ? wsum[lane] : 0;
    const int si = wave_inclusive_scan(s);
    if (lane < nw) wsum[lane] = si - s;
    if (lane == nw - 1) a[n] = si;
  }
  __syncthreads();
  int run = wsum[w] + inc - local;
  for (int i = lo; i < hi; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  __syncthreads();
}

struct LayoutOut {  // the batch-wide outputs, written by rank workgroup 0
  int32_t *expert_count, *expert_off, *rank_count, *rank_off,
      *rank_token_count, *node_count, *node_off;
};

// Expert and node totals (ebase[0..E), nbase[0..N) in LDS) to global
// exclusive offsets, in place (ebase[E], nbase[N] get the totals); rank
// workgroup 0 also writes the batch-wide outputs.  Ends with a barrier.
__device__ void offsets_from_totals(int32_t *ebase, int32_t *nbase, int E,
                                    int R, int N, int per_rank,
                                    const int32_t *tail, const LayoutOut &lo,
                                    int32_t *wsum) {
  // wave 0 scans the node totals (N <= 64) in registers while the
  // workgroup scans the expert totals
  int nv = 0, ni = 0;
  if (threadIdx.x < kWave) {
    nv = (int)threadIdx.x < N ? nbase[threadIdx.x] : 0;
    ni = wave_inclusive_scan(nv);
  }
  scan_inplace(ebase, E, wsum);  // ends with a barrier
  if ((int)threadIdx.x < N) nbase[threadIdx.x] = ni - nv;
  if ((int)threadIdx.x == N - 1) nbase[N] = ni;
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      lo.expert_count[e] = ebase[e + 1] - ebase[e];
      lo.expert_off[e] = ebase[e];
    }
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
      lo.rank_off[r] = ebase[r * per_rank];
      lo.rank_count[r] = ebase[(r + 1) * per_rank] - ebase[r * per_rank];
      if (lo.rank_token_count) lo.rank_token_count[r] = tail[E + r];
    }
    for (int n = threadIdx.x; n <= N; n += blockDim.x) {
      if (lo.node_count && n < N) lo.node_count[n] = nbase[n + 1] - nbase[n];
      if (lo.node_off) lo.node_off[n] = nbase[n];
    }
    if (threadIdx.x == 0) {
      lo.expert_off[E] = ebase[E];
      lo.rank_off[R] = ebase[E];
    }
  }
  __syncthreads();
}

constexpr int kRankRowRegs = 8;  // table values a thread loads at once
// Up to this many tiles and columns the rank kernel reads the raw per-tile
// counts itself (MODE 2) and no scan launch runs.
constexpr int kFoldTiles = 64;
constexpr int kFoldCols = 64;

constexpr int kFoldBatch = 8;  // columns whose loads go out together

// MODE 0: the tail row of the table holds the global offsets (the
// one-workgroup scan wrote them and the batch-wide outputs).  MODE 1: the
// tail row holds each column's total (the column-parallel scan): every
// workgroup turns the expert and node totals into global exclusive offsets
// in LDS (workgroup 0 also writes the batch-wide outputs), then adds its
// tile's prefixes.  MODE 2: the table holds the raw per-tile counts (at
// most kFoldTiles rows of kFoldCols): wave 0, lane r holding tile r, sums
// every column over all tiles and over the tiles before this one, and the
// rest is as in MODE 1.
template <int KM, int MODE>
__global__ __launch_bounds__(1024) void layout_rank_kernel(
    const int32_t *__restrict__ idx, int T, int K, int E, int R, int N,
    int per_rank, uint32_t m_node, const int32_t *__restrict__ table,
    LayoutOut lo, int32_t *__restrict__ slot_pos,
    int32_t *__restrict__ row_src, int32_t *__restrict__ node_slot) {
  extern __shared__ uint64_t sm[];
  const int cr = E + N;  // expert bitmaps, then node bitmaps
  const int cols = E + R + N;
  const int W = blockDim.x / kWave;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  int ev[KM];
  if (t < T) load_ids<KM>(idx + (size_t)t * K, K, ev);
  uint64_t *bm = sm;                                  // [W][cr]
  int32_t *ebase = (int32_t *)(sm + (size_t)W * cr);  // [E + 1]
  int32_t *nbase = ebase + E + 1;                     // [N + 1]
  int32_t *wsum = nbase + N + 1;                      // [16]
  for (int i = threadIdx.x; i < W * cr; i += blockDim.x) bm[i] = 0;
  const int32_t *tile = table + (size_t)blockIdx.x * cols;
  const int32_t *tail = table + (size_t)gridDim.x * cols;
  // The expert and node columns (value j < E + N: column j, or E + R + j - E
  // for a node) of the tail row and of the tile's row.  The first
  // kRankRowRegs * B of each are loaded together, with the ids, into
  // registers (a loop of loads and LDS stores waits for each load in turn:
  // that was 1.4 us for DeepSeek-V3 and 3.3 us for Kimi K2 before the
  // offsets could start, and as much again for the tile's row); the rest,
  // for very wide tables only, in a loop.
  const int B = blockDim.x;
  if constexpr (MODE == 2) {
    __shared__ int32_t ftot[kFoldCols], fpre[kFoldCols];
    if (threadIdx.x < kWave) {  // wave 0: lane r holds tile r
      // one inclusive scan over the tiles per column: its last lane is the
      // column's total, lane b less b's own count this tile's prefix
      const int b = blockIdx.x;
      for (int c0 = 0; c0 < cols; c0 += kFoldBatch) {
        int v[kFoldBatch];
#pragma unroll
        for (int u = 0; u < kFoldBatch; ++u)
          v[u] = lane < (int)gridDim.x && c0 + u < cols
                     ? table[(size_t)lane * cols + c0 + u]
                     : 0;
#pragma unroll
        for (int u = 0; u < kFoldBatch; ++u) {
          if (c0 + u < cols) {  // uniform
            const int inc = wave_inclusive_scan(v[u]);
            const int all = __builtin_amdgcn_readlane(inc, kWave - 1);
            const int pre = __builtin_amdgcn_readlane(inc, b) -
                            __builtin_amdgcn_readlane(v[u], b);
            if (lane == 0) {
              ftot[c0 + u] = all;
              fpre[c0 + u] = pre;
            }
          }
        }
      }
    }
    __syncthreads();
    for (int j = threadIdx.x; j < cr; j += B)
      ebase[j < E ? j : j + 1] = ftot[j < E ? j : j + R];
    __syncthreads();
    offsets_from_totals(ebase, nbase, E, R, N, per_rank, ftot, lo, wsum);
    for (int j = threadIdx.x; j < cr; j += B)
      ebase[j < E ? j : j + 1] += fpre[j < E ? j : j + R];
    __syncthreads();
  } else {
  int tl[kRankRowRegs], tv[kRankRowRegs];
#pragma unroll
  for (int u = 0; u < kRankRowRegs; ++u) {
    const int j = u * B + threadIdx.x;
    const int col = j < E ? j : j + R;
    tl[u] = j < cr ? tail[col] : 0;
    tv[u] = j < cr ? tile[col] : 0;
  }
#pragma unroll
  for (int u = 0; u < kRankRowRegs; ++u) {
    const int j = u * B + threadIdx.x;
    if (j < cr) ebase[j < E ? j : j + 1] = tl[u];  // nbase = ebase + E + 1
  }
  for (int j = kRankRowRegs * B + threadIdx.x; j < cr; j += B)
    ebase[j < E ? j : j + 1] = tail[j < E ? j : j + R];
  __syncthreads();
  if constexpr (MODE == 1) offsets_from_totals(ebase, nbase, E, R, N,
                                               per_rank, tail, lo, wsum);
#pragma unroll
  for (int u = 0; u < kRankRowRegs; ++u) {
    const int j = u * B + threadIdx.x;
    if (j < cr) ebase[j < E ? j : j + 1] += tv[u];
  }
  for (int j = kRankRowRegs * B + threadIdx.x; j < cr; j += B)
    ebase[j < E ? j : j + 1] += tile[j < E ? j : j + R];
  __syncthreads();
  }

  const uint64_t bit = 1ull << lane;
  const uint64_t below = bit - 1;
  uint64_t *mine = bm + (size_t)w * cr;
  uint64_t mask = 0;
  if (t < T) {
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k >= K) break;
      const int e = ev[k];
      if ((unsigned)e >= (unsigned)E) continue;
      atomicOr((unsigned long long *)&mine[e], bit);
      mask |= 1ull << div_small(e, m_node);
    }
    if (node_slot)
      for (uint64_t m = mask; m; m &= m - 1)
        atomicOr((unsigned long long *)&mine[E + __ffsll((long long)m) - 1],
                 bit);
  }
  __syncthreads();
  if (t >= T) return;

  // every slot's rank first (LDS reads only), then the stores; the two
  // fully unrolled passes keep ev and sp in registers for every KM
  int sp[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int e = ev[k];
    int s = -1;
    if (k < K && (unsigned)e < (unsigned)E) {
      s = ebase[e] + __popcll(mine[e] & below);
      for (int v = 0; v < w; ++v) s += __popcll(bm[(size_t)v * cr + e]);
    }
    sp[k] = s;
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k < K) {
      const size_t i = (size_t)t * K + k;
      slot_pos[i] = sp[k];
      if (sp[k] >= 0) row_src[sp[k]] = (int32_t)i;
    }
  }
  if (node_slot) {
    for (int n = 0; n < N; ++n) {
      int s = -1;
      if (mask >> n & 1) {
        s = nbase[n] + __popcll(mine[E + n] & below);
        for (int v = 0; v < w; ++v) s += __popcll(bm[(size_t)v * cr + E + n]);
      }
      node_slot[(size_t)t * N + n] = s;
    }
  }
}

// The whole layout in one workgroup of 1024 threads when every token fits
// in one tile (the decode case): one launch instead of three.  Thread t
// takes token t; the 64 tokens t/64 = p share wave bitmap p.  Once the
// bitmaps are built, thread c turns column c into prefix counts over p,
// which give every rank directly: rank of (t, e) = expert offset + tokens
// of e in bitmaps before p + popcount(bitmap p & lanes below).  (The same
// kernel with 4 tokens per thread, for up to 4096 tokens, was slower than
// the three launches for the Mixtral shape: 20.5 vs 14.6 us; one CU issues
// every store.)
template <int KM>
__global__ __launch_bounds__(1024) void layout_block_kernel(
    const int32_t *__restrict__ idx, int T, int K, int E, int R, int N,
    int per_rank, uint32_t m_rank, uint32_t m_node,
    int32_t *__restrict__ expert_count,
    int32_t *__restrict__ expert_off, int32_t *__restrict__ rank_count,
    int32_t *__restrict__ rank_off, int32_t *__restrict__ rank_token_count,
    uint64_t *__restrict__ node_mask, int32_t *__restrict__ node_count,
    int32_t *__restrict__ node_off, int32_t *__restrict__ node_slot,
    int32_t *__restrict__ slot_pos, int32_t *__restrict__ row_src,
    int32_t *__restrict__ err) {
  extern __shared__ uint64_t bm[];  // [P][cols], then the int32 arrays
  const int cols = E + R + N;
  const int P = (T + kWave - 1) / kWave;  // bitmaps, <= 16
  const int B = blockDim.x;
  const int lane = threadIdx.x % kWave;
  int32_t *pfx = (int32_t *)(bm + (size_t)P * cols);  // [P][cols]
  int32_t *tot = pfx + (size_t)P * cols;               // [cols]
  int32_t *eoff = tot + cols;                          // [E + 1]
  int32_t *noff = eoff + E + 1;                        // [N + 1]
  const uint64_t bit = 1ull << lane;
  const uint64_t below = bit - 1;
  const int t = threadIdx.x;
  int ev[KM];
  if (t < T) load_ids<KM>(idx + (size_t)t * K, K, ev);
  for (int i = threadIdx.x; i < P * cols; i += B) bm[i] = 0;
  __syncthreads();

  int bad = 0;
  if (t < T) {  // set the bitmaps' bits
    uint64_t *mine = bm + (size_t)(t / kWave) * cols;
    uint64_t mask = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k >= K) break;
      const int e = ev[k];
      if ((unsigned)e >= (unsigned)E) {
        bad |= MOE_DEVERR_EXPERT_RANGE;
        continue;
      }
      const uint64_t old = atomicOr((unsigned long long *)&mine[e], bit);
      if (old & bit) bad |= MOE_DEVERR_DUP_EXPERT;
      atomicOr((unsigned long long *)&mine[E + div_small(e, m_rank)], bit);
      mask |= 1ull << div_small(e, m_node);
    }
    for (uint64_t m = mask; m; m &= m - 1)
      atomicOr((unsigned long long *)&mine[E + R + __ffsll((long long)m) - 1],
               bit);
    if (node_mask) node_mask[t] = mask;
  }
  raise_error(err, bad);
  __syncthreads();

  for (int c = threadIdx.x; c < cols; c += B) {  // prefix counts over p
    int run = 0;
#pragma unroll 8
    for (int q = 0; q < P; ++q) {
      const int x = __popcll(bm[(size_t)q * cols + c]);
      pfx[(size_t)q * cols + c] = run;
      run += x;
    }
    tot[c] = run;
  }
  __syncthreads();
  block_exclusive_scan(tot, E, eoff);  // ends with a barrier
  for (int e = threadIdx.x; e < E; e += B) {
    expert_count[e] = tot[e];
    expert_off[e] = eoff[e];
  }
  for (int r = threadIdx.x; r < R; r += B) {
    rank_off[r] = eoff[r * per_rank];
    rank_count[r] = eoff[(r + 1) * per_rank] - eoff[r * per_rank];
    if (rank_token_count) rank_token_count[r] = tot[E + r];
  }
  if (threadIdx.x == 0) {
    expert_off[E] = eoff[E];
    rank_off[R] = eoff[E];
    int run = 0;
    for (int n = 0; n < N; ++n) {
      noff[n] = run;
      if (node_count) node_count[n] = tot[E + R + n];
      if (node_off) node_off[n] = run;
      run += tot[E + R + n];
    }
    noff[N] = run;
    if (node_off) node_off[N] = run;
  }
  __syncthreads();

  if (t < T) {  // the ranks
    const size_t p = t / kWave;
    const uint64_t *mine = bm + p * cols;
    const int32_t *before = pfx + p * cols;
    int sp[KM];
    uint64_t mask = 0;
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      const int e = ev[k];
      int s = -1;
      if (k < K && (unsigned)e < (unsigned)E) {
        s = eoff[e] + before[e] + __popcll(mine[e] & below);
        mask |= 1ull << div_small(e, m_node);
      }
      sp[k] = s;
    }
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < K) {
        const size_t i = (size_t)t * K + k;
        slot_pos[i] = sp[k];
        if (sp[k] >= 0) row_src[sp[k]] = (int32_t)i;
      }
    }
    if (node_slot) {
      for (int n = 0; n < N; ++n) {
        const int c = E + R + n;
        node_slot[(size_t)t * N + n] =
            (mask >> n & 1)
                ? noff[n] + before[c] + __popcll(mine[c] & below)
                : -1;
      }
    }
  }
}

}  // namespace

size_t rank_lds_bytes(const moe_cfg &c, int w) {
  return (size_t)w * (c.E + c.N) * 8 + (size_t)(c.E + c.N + 18) * 4;
}

// Default tokens per layout tile.  More tiles spread the count and rank
// kernels over more CUs; each tile also adds one table row to the column
// scan and one more workgroup to drain.  Measured on the model shapes, the
// layout is fastest near 128 tiles, so the tile starts at 256 tokens and
// halves (down to 64) while it leaves fewer than 91 tiles, the count nearest
// 128 on a log scale.  A smaller tile is taken only while the table stays
// within 256 KiB, which keeps the workspace of wide configurations small.
// Up to 256 tokens the single tile stays: one workgroup then does the whole
// layout.
static int default_layout_tile(const moe_cfg &c, int cols) {
  int tile = kDefaultLayoutTile;
  if (c.T <= tile) return tile;
  while (tile > kMinDefaultLayoutTile) {
    if ((c.T + tile - 1) / tile >= kLayoutTileCountFloor) break;
    const int half = tile / 2;
    const size_t rows = (size_t)(c.T + half - 1) / half + 1;
    if (rows * cols * 4 > kLayoutShrinkTableMax) break;
    tile = half;
  }
  return tile;
}

LayoutGeom layout_geom(const moe_cfg &c) {
  LayoutGeom g{};
  g.cols = c.E + c.R + c.N;
  const int want = c.layout_tile ? c.layout_tile : default_layout_tile(c, g.cols);
  int w = want / kWave;
  // count kernel: W*cols*8 bytes; rank kernel: W*(E+N)*8 + (E+N+18)*4
  while (w > 1 && ((size_t)w * g.cols * 8 > (size_t)kLdsBudget ||
                   rank_lds_bytes(c, w) > (size_t)kLdsBudget))
    w >>= 1;
  g.tile_waves = w;
  g.tile_tokens = w * kWave;
  g.nblocks = (c.T + g.tile_tokens - 1) / g.tile_tokens;
  // one spare tail row after the per-tile rows carries the column totals
  g.table_bytes = ((size_t)(g.nblocks + 1) * g.cols * 4 + 255) & ~(size_t)255;
  g.ws_bytes = kWsHeader + g.table_bytes;
  return g;
}

namespace {

// The scan and rank launches, once the count table's rows [0, nblocks) and
// node_mask hold the per-tile counts (from layout_count_kernel, or from the
// gate's fused count pass).
template <int KM>
hipError_t launch_layout_tail(const moe_cfg &c, const int32_t *topk_idx,
                              const moe_layout &lay, void *ws,
                              hipStream_t stream) {
  const LayoutGeom g = layout_geom(c);
  int32_t *table = (int32_t *)((char *)ws + kWsHeader);
  const int per_rank = c.E / c.R;
  const uint32_t m_node = div_magic(c.E / c.N);
  const int threads = g.tile_tokens;
  const LayoutOut lo{lay.expert_count, lay.expert_off, lay.rank_count,
                     lay.rank_off, lay.rank_token_count, lay.node_count,
                     lay.node_off};
  const size_t rank_lds = rank_lds_bytes(c, g.tile_waves);
  if (g.nblocks >= 1 && g.nblocks <= kFoldTiles && g.cols <= kFoldCols) {
    // a small table: every rank workgroup sums the raw counts itself
    hipLaunchKernelGGL((layout_rank_kernel<KM, 2>), dim3(g.nblocks),
                       dim3(threads), rank_lds, stream, topk_idx, c.T, c.K,
                       c.E, c.R, c.N, per_rank, m_node, table, lo,
                       lay.slot_pos, lay.row_src, lay.node_slot);
    return hipGetLastError();
  }
  if (g.nblocks <= kSmallTable) {
    // One workgroup scans the few tile rows (rows [0, nblocks) become
    // exclusive prefixes, the tail row the global offsets) and writes the
    // batch-wide outputs; with no tokens that is all there is to do.
    const size_t lds = (size_t)(g.cols + c.E + 1) * 4;
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(1024), lds, stream,
                       table, g.nblocks, c.E, c.R, c.N, per_rank,
                       lay.expert_count, lay.expert_off, lay.rank_count,
                       lay.rank_off, lay.rank_token_count, lay.node_count,
                       lay.node_off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || g.nblocks == 0) return e;
    hipLaunchKernelGGL((layout_rank_kernel<KM, 0>), dim3(g.nblocks),
                       dim3(threads), rank_lds, stream, topk_idx, c.T, c.K,
                       c.E, c.R, c.N, per_rank, m_node, table, lo,
                       lay.slot_pos, lay.row_src, lay.node_slot);
    return hipGetLastError();
  }
  // Many tiles: the column-parallel scan (per-tile exclusive prefixes,
  // column totals in the tail row), and every rank workgroup derives the
  // global offsets from the totals.
  hipLaunchKernelGGL(layout_scan_cols_kernel,
                     dim3((g.cols + kScanCols - 1) / kScanCols),
                     dim3(kScanCols * kScanChunks), 0, stream, table,
                     g.nblocks, g.cols);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((layout_rank_kernel<KM, 1>), dim3(g.nblocks),
                     dim3(threads), rank_lds, stream, topk_idx, c.T, c.K, c.E,
                     c.R, c.N, per_rank, m_node, table, lo, lay.slot_pos,
                     lay.row_src, lay.node_slot);
  return hipGetLastError();
}

template <int KM>
hipError_t launch_layout_km(const moe_cfg &c, const int32_t *topk_idx,
                            const moe_layout &lay, void *ws,
                            hipStream_t stream) {
  const LayoutGeom g = layout_geom(c);
  int32_t *err = (int32_t *)ws;
  int32_t *table = (int32_t *)((char *)ws + kWsHeader);
  const int per_rank = c.E / c.R;
  const uint32_t m_rank = div_magic(per_rank);
  const uint32_t m_node = div_magic(c.E / c.N);
  const int threads = g.tile_tokens;

  if (g.nblocks == 1) {
    // every token in one tile: one workgroup does the whole layout
    const int P = (c.T + kWave - 1) / kWave;
    const size_t lds = (size_t)P * g.cols * 12 +
                       (size_t)(g.cols + c.E + 1 + c.N + 1) * 4;
    if (lds <= (size_t)kLdsBudget) {
      hipLaunchKernelGGL((layout_block_kernel<KM>), dim3(1), dim3(1024),
                         lds, stream, topk_idx, c.T, c.K, c.E, c.R, c.N,
                         per_rank, m_rank, m_node, lay.expert_count,
                         lay.expert_off, lay.rank_count, lay.rank_off,
                         lay.rank_token_count, lay.node_mask, lay.node_count,
                         lay.node_off, lay.node_slot, lay.slot_pos,
                         lay.row_src, err);
      return hipGetLastError();
    }
  }
  if (g.nblocks > 0) {
    const size_t lds = (size_t)g.tile_waves * g.cols * 8;
    hipLaunchKernelGGL(layout_count_kernel<KM>, dim3(g.nblocks), dim3(threads),
                       lds, stream, topk_idx, c.T, c.K, c.E, c.R, c.N,
                       m_rank, m_node, lay.node_mask, table, err);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_layout_tail<KM>(c, topk_idx, lay, ws, stream);
}

}  // namespace

hipError_t launch_layout(const moe_cfg &c, const int32_t *topk_idx,
                         const moe_layout &lay, void *ws,
                         hipStream_t stream) {
  if (c.K <= 4) return launch_layout_km<4>(c, topk_idx, lay, ws, stream);
  if (c.K <= 8) return launch_layout_km<8>(c, topk_idx, lay, ws, stream);
  if (c.K <= 16) return launch_layout_km<16>(c, topk_idx, lay, ws, stream);
  return launch_layout_km<32>(c, topk_idx, lay, ws, stream);  // K <= 32
}

hipError_t launch_layout_after_count(const moe_cfg &c,
                                     const int32_t *topk_idx,
                                     const moe_layout &lay, void *ws,
                                     hipStream_t stream) {
  if (c.K <= 4) return launch_layout_tail<4>(c, topk_idx, lay, ws, stream);
  if (c.K <= 8) return launch_layout_tail<8>(c, topk_idx, lay, ws, stream);
  if (c.K <= 16) return launch_layout_tail<16>(c, topk_idx, lay, ws, stream);
  return launch_layout_tail<32>(c, topk_idx, lay, ws, stream);
}

}  // namespace moe
