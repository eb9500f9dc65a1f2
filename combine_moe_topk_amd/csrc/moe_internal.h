// Internal declarations shared by the host API and the kernel translation
// units of the MI355X MoE dispatch/combine library.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_topk.h"

namespace moe {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr size_t kWsHeader = 256;    // workspace header: error word + pad
constexpr int kLdsBudget = 65536;    // bytes of LDS a layout workgroup may use
constexpr int kDefaultLayoutTile = 256;    // largest default layout tile
constexpr int kMinDefaultLayoutTile = 64;  // smallest default layout tile
constexpr int kLayoutTileCountFloor = 91;  // default tile halves below this
constexpr size_t kLayoutShrinkTableMax = 256 << 10;  // bytes
constexpr int kMaxLevels = MOE_MAX_LEVELS;  // capacity / bucket levels

// 16-byte vector used for every row copy (one global_load/store_dwordx4).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Quotient n / d for 0 <= n, d and n * d < 2^31 (expert ids and experts per
// rank or node, both at most 4096) as one 32x32->64 multiply and a shift, in
// place of the dozen-instruction division sequence a runtime divisor costs.
// With m = ceil(2^31 / d) = 2^31 / d + f (0 <= f < 1) and n = q d + r:
// n m / 2^31 = q + r / d + n f / 2^31 < q + (d - 1) / d + 1 / d = q + 1.
inline uint32_t div_magic(int d) {
  return (uint32_t)(((1ull << 31) + (uint64_t)d - 1) / (uint64_t)d);
}
__device__ __forceinline__ int div_small(int n, uint32_t m) {
  return (int)(((uint64_t)(uint32_t)n * m) >> 31);
}

// Launch geometry of the three layout kernels.  A layout workgroup owns a
// tile of `tile_tokens` consecutive tokens, one token per lane, and keeps one
// 64-bit token bitmap per (wave, expert / rank / node) in LDS.
struct LayoutGeom {
  int tile_waves;   // waves per workgroup
  int tile_tokens;  // tile_waves * 64
  int nblocks;      // ceil(T / tile_tokens)
  int cols;         // E + R + N count columns per workgroup
  size_t table_bytes;
  size_t ws_bytes;  // header + nblocks * cols int32 (256-byte rounded)
};

LayoutGeom layout_geom(const moe_cfg &c);

hipError_t launch_fill_u32(uint32_t *p, uint32_t value, size_t n,
                           hipStream_t stream);

// The fused call's host checks (cfg, layout and row pointers; not the
// workspace) and its launch sequence gate -> layout -> pack -> combine, the
// combine reading send.  ws holds layout_geom(c).ws_bytes.
int check_fused(const moe_cfg *cfg, const void *x, const float *logits,
                const int32_t *topk_idx, const float *topk_w,
                const moe_layout *layout, const void *send, const void *out);
hipError_t launch_fused(const moe_cfg &c, const void *x, const float *logits,
                        const float *expert_scale, int32_t *topk_idx,
                        float *topk_w, const moe_layout &lay, void *send,
                        void *out, void *ws, hipStream_t stream);

hipError_t launch_gate(const moe_cfg &c, const float *logits,
                       int32_t *topk_idx, float *topk_w, hipStream_t stream);

hipError_t launch_layout(const moe_cfg &c, const int32_t *topk_idx,
                         const moe_layout &lay, void *ws, hipStream_t stream);

// The layout's scan and rank launches alone (layout.hip), for when the
// count table rows [0, nblocks) and node_mask already hold the per-tile
// counts that its count launch would write.
hipError_t launch_layout_after_count(const moe_cfg &c,
                                     const int32_t *topk_idx,
                                     const moe_layout &lay, void *ws,
                                     hipStream_t stream);

// The gate and the layout's count launch as one launch (gate.hip): the
// gate's picks plus the count table rows and node_mask, as launch_gate and
// then the count launch of launch_layout would leave them.  gate_count_ok:
// the gate takes 16 lanes a token and the layout has more than one tile of
// at most 128 tokens (a workgroup runs the gate of 64 tokens at a time).
bool gate_count_ok(const moe_cfg &c);
hipError_t launch_gate_count(const moe_cfg &c, const float *logits,
                             int32_t *topk_idx, float *topk_w,
                             uint64_t *node_mask, void *ws,
                             hipStream_t stream);

// send-style copy: dst[slots[t*W + w]] = x[t] for w < W (W <= 64), entries
// outside [0, rows) skipped; row_bytes a multiple of 16.
hipError_t launch_pack_rows(const void *x, const int32_t *slots, int W,
                            int rows, void *dst, int T, int row_bytes,
                            hipStream_t stream);

hipError_t launch_pack(const moe_cfg &c, const void *x,
                       const int32_t *slot_pos, void *send,
                       hipStream_t stream);

// rows: rows of y (slots outside [0, rows) add 0); -1 means T*K.
hipError_t launch_combine(const moe_cfg &c, const void *y,
                          const int32_t *slot_pos, const float *topk_w,
                          const int32_t *topk_idx, const float *expert_scale,
                          void *out, hipStream_t stream, int rows = -1);

// Decode-sized fused step (decode.hip): layout, pack and combine of a small
// batch in one launch after the gate, the same results as the layout, pack
// and combine kernels.  decode_ok: the batch fits (1 <= T <= 1024, T*K <=
// 4096, its LDS tables within 64 KiB).
bool decode_ok(const moe_cfg &c);
hipError_t launch_decode(const moe_cfg &c, const void *x,
                         const int32_t *topk_idx, const float *topk_w,
                         const float *expert_scale, const moe_layout &lay,
                         void *send, void *out, hipStream_t stream);

// Node-level two-leg dispatch and hierarchical combine (nodes.hip).  Leg-1
// and partial buffers hold node_rows_max(c) = T * min(K, N) rows.
int node_rows_max(const moe_cfg &c);

hipError_t launch_pack_nodes(const moe_cfg &c, const void *x,
                             const int32_t *node_slot, void *node_send,
                             hipStream_t stream);

hipError_t launch_forward(const moe_cfg &c, const void *node_send,
                          const int32_t *node_slot, const int32_t *topk_idx,
                          const int32_t *slot_pos, void *send,
                          hipStream_t stream);

hipError_t launch_partial(const moe_cfg &c, const void *y,
                          const int32_t *slot_pos, const float *topk_w,
                          const int32_t *topk_idx, const float *expert_scale,
                          const int32_t *node_slot, int part_dtype,
                          void *part, hipStream_t stream);

hipError_t launch_sum_nodes(const moe_cfg &c, const void *part, int part_dtype,
                            const int32_t *node_slot, void *out,
                            hipStream_t stream);

// FP8 (E4M3) dispatch with per-block scales (fp8.hip).  Rows are H codes,
// H/B fp32 scales, zero padding to a multiple of 128 bytes:
// round_up(H + 4H/B, 128) bytes a row.
size_t fp8_row_bytes(int H, int B);
bool fp8_block_ok(const moe_cfg &c, int B);

hipError_t launch_pack_fp8(const moe_cfg &c, int B, const void *x,
                           const int32_t *slot_pos, void *send,
                           hipStream_t stream);

hipError_t launch_combine_fp8(const moe_cfg &c, int B, const void *y,
                              const int32_t *slot_pos, const float *topk_w,
                              const int32_t *topk_idx,
                              const float *expert_scale, void *out,
                              hipStream_t stream);

// Capacity-padded and bucketed layout (capacity.hip).
bool levels_ok(const moe_cfg &c, const int32_t *levels, int q);
size_t capacity_ws_bytes(const moe_cfg &c);

hipError_t launch_layout_capacity(const moe_cfg &c, const int32_t *topk_idx,
                                  const int32_t *levels, int q,
                                  const moe_capacity_layout &cl, void *ws,
                                  hipStream_t stream);

hipError_t launch_pack_capacity(const moe_cfg &c, const void *x,
                                const int32_t *slot_pos,
                                const int32_t *row_src, int n_rows,
                                void *send, hipStream_t stream);

// Communication-aware task assignment (assign.hip).
size_t assign_ws_bytes(const moe_cfg &c);
constexpr int kMaxAssignNodes = 24;  // nodes the cover search accepts
bool assign_ok(const moe_cfg &c);  // N <= 24 nodes, R/N <= 64 ranks a node

hipError_t launch_assign(const moe_cfg &c, const int32_t *topk_idx,
                         const int32_t *src_rank, const uint8_t *holds,
                         const uint32_t *u_node, const uint32_t *u_rank,
                         int32_t *assign_rank, uint64_t *remote_mask, void *ws,
                         hipStream_t stream);

}  // namespace moe
