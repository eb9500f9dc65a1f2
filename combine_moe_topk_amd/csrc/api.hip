// Host side of the C ABI declared in include/moe_topk.h: argument validation,
// workspace sizing, launch sequencing and error capture.  No call allocates,
// synchronises (except moe_read_device_error) or keeps state between calls.
#include <string.h>

#include "moe_internal.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int validate(const moe_cfg *c) {
  if (!c) return MOE_EINVAL;
  if (c->T < 0 || c->H < 1 || c->E < 1 || c->K < 1 || c->R < 1 || c->N < 1)
    return MOE_EINVAL;
  if (c->K > c->E || c->K > 32) return MOE_EINVAL;
  if (c->E > 4096) return MOE_EINVAL;
  if (c->E % c->R != 0 || c->R % c->N != 0 || c->N > 64) return MOE_EINVAL;
  if ((int64_t)c->T * c->K > INT32_MAX) return MOE_EINVAL;
  // headroom for int token indexes rounded up to a whole tile (1024)
  if (c->T > INT32_MAX - 4096) return MOE_EINVAL;
  switch (c->layout_tile) {
    case 0: case 64: case 128: case 256: case 512: case 1024: break;
    default: return MOE_EINVAL;
  }
  if ((c->flags & ~MOE_F_NO_RENORM) != 0) return MOE_EINVAL;
  if (c->x_dtype != MOE_F32 && c->x_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (c->out_dtype != MOE_F32 && c->out_dtype != MOE_BF16)
    return MOE_EUNSUPPORTED;
  if (c->H % 8 != 0) return MOE_EUNSUPPORTED;  // rows move in 8-element units
  // one layout wave's LDS bitmaps must fit (see layout_geom)
  if ((size_t)(c->E + c->R + c->N) * 8 > (size_t)moe::kLdsBudget ||
      (size_t)(c->E + c->N) * 12 > (size_t)moe::kLdsBudget)
    return MOE_EUNSUPPORTED;
  if ((size_t)(c->E + c->R + c->N + c->E + 1) * 4 > (size_t)moe::kLdsBudget)
    return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

int check_layout_ptrs(const moe_cfg *c, const moe_layout *l) {
  if (!l) return MOE_EINVAL;
  if (!l->expert_count || !l->expert_off || !l->rank_count || !l->rank_off)
    return MOE_EINVAL;
  if (c->T > 0 && (!l->slot_pos || !l->row_src)) return MOE_EINVAL;
  if (l->node_mask && !aligned(l->node_mask, 8)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int check_ws(const moe_cfg *c, const void *ws, size_t ws_bytes) {
  if (!ws) return MOE_EWORKSPACE;
  if (!aligned(ws, 256)) return MOE_EUNSUPPORTED;
  if (ws_bytes < moe::layout_geom(*c).ws_bytes) return MOE_EWORKSPACE;
  return MOE_OK;
}

__global__ void fill_u32_kernel(uint32_t *p, uint32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

namespace moe {

int check_fused(const moe_cfg *cfg, const void *x, const float *logits,
                const int32_t *topk_idx, const float *topk_w,
                const moe_layout *layout, const void *send, const void *out) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if ((rc = check_layout_ptrs(cfg, layout)) != MOE_OK) return rc;
  if (cfg->T > 0) {
    if (!x || !logits || !topk_idx || !topk_w || !send || !out)
      return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(send) || !aligned16(out))
      return MOE_EUNSUPPORTED;
  }
  return MOE_OK;
}

hipError_t launch_fused(const moe_cfg &c, const void *x, const float *logits,
                        const float *expert_scale, int32_t *topk_idx,
                        float *topk_w, const moe_layout &lay, void *send,
                        void *out, void *ws, hipStream_t stream) {
  hipError_t e;
  if (!decode_ok(c) && gate_count_ok(c)) {
    // the gate also writes the layout's per-tile counts: one launch fewer,
    // and the ids are not read back for counting
    e = launch_gate_count(c, logits, topk_idx, topk_w, lay.node_mask, ws,
                          stream);
    if (e == hipSuccess)
      e = launch_layout_after_count(c, topk_idx, lay, ws, stream);
  } else {
    e = launch_gate(c, logits, topk_idx, topk_w, stream);
    if (e != hipSuccess) return e;
    // a decode-sized batch: layout, pack and combine in one launch
    if (decode_ok(c))
      return launch_decode(c, x, topk_idx, topk_w, expert_scale, lay, send,
                           out, stream);
    e = launch_layout(c, topk_idx, lay, ws, stream);
  }
  if (e == hipSuccess) e = launch_pack(c, x, lay.slot_pos, send, stream);
  if (e == hipSuccess)
    e = launch_combine(c, send, lay.slot_pos, topk_w, topk_idx, expert_scale,
                       out, stream);
  return e;
}

hipError_t launch_fill_u32(uint32_t *p, uint32_t value, size_t n,
                           hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid), dim3(256), 0, stream, p,
                     value, n);
  return hipGetLastError();
}
}  // namespace moe

extern "C" {

int moe_validate_cfg(const moe_cfg *cfg) { return validate(cfg); }

size_t moe_workspace_bytes(const moe_cfg *cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return moe::layout_geom(*cfg).ws_bytes;
}

int moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || ws_bytes < moe::kWsHeader) return MOE_EWORKSPACE;
  if (!aligned(ws, 256)) return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_fill_u32(
      (uint32_t *)ws, 0u, moe::kWsHeader / 4, stream));
}

int moe_topk_gate(const moe_cfg *cfg, const float *logits, int32_t *topk_idx,
                  float *topk_w, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->T > 0 && (!logits || !topk_idx || !topk_w)) return MOE_EINVAL;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
    return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_gate(*cfg, logits, topk_idx, topk_w, stream));
}

int moe_dispatch_layout(const moe_cfg *cfg, const int32_t *topk_idx,
                        const moe_layout *layout, void *ws, size_t ws_bytes,
                        hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->T > 0 && !topk_idx) return MOE_EINVAL;
  if ((rc = check_layout_ptrs(cfg, layout)) != MOE_OK) return rc;
  if ((rc = check_ws(cfg, ws, ws_bytes)) != MOE_OK) return rc;
  return launch_status(moe::launch_layout(*cfg, topk_idx, *layout, ws, stream));
}

int moe_dispatch_pack(const moe_cfg *cfg, const void *x,
                      const int32_t *slot_pos, void *send,
                      hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !slot_pos || !send) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(send) || !aligned(slot_pos, 4))
    return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_pack(*cfg, x, slot_pos, send, stream));
}

int moe_combine(const moe_cfg *cfg, const void *y, const int32_t *slot_pos,
                const float *topk_w, const int32_t *topk_idx,
                const float *expert_scale, void *out, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->T == 0) return MOE_OK;
  if (!y || !slot_pos || !topk_w || !out) return MOE_EINVAL;
  if (expert_scale && !topk_idx) return MOE_EINVAL;
  if (!aligned16(y) || !aligned16(out)) return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_combine(*cfg, y, slot_pos, topk_w, topk_idx,
                                           expert_scale, out, stream));
}

int moe_dispatch_combine(const moe_cfg *cfg, const void *x,
                         const float *logits, const float *expert_scale,
                         int32_t *topk_idx, float *topk_w,
                         const moe_layout *layout, void *send, void *out,
                         void *ws, size_t ws_bytes, hipStream_t stream) {
  int rc = moe::check_fused(cfg, x, logits, topk_idx, topk_w, layout, send,
                            out);
  if (rc != MOE_OK) return rc;
  if ((rc = check_ws(cfg, ws, ws_bytes)) != MOE_OK) return rc;
  return launch_status(moe::launch_fused(*cfg, x, logits, expert_scale,
                                         topk_idx, topk_w, *layout, send, out,
                                         ws, stream));
}

size_t moe_node_rows_max(const moe_cfg *cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return (size_t)moe::node_rows_max(*cfg);
}

int moe_dispatch_pack_nodes(const moe_cfg *cfg, const void *x,
                            const int32_t *node_slot, void *node_send,
                            hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !node_slot || !node_send) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(node_send) || !aligned(node_slot, 4))
    return MOE_EUNSUPPORTED;
  return launch_status(
      moe::launch_pack_nodes(*cfg, x, node_slot, node_send, stream));
}

int moe_dispatch_forward(const moe_cfg *cfg, const void *node_send,
                         const int32_t *node_slot, const int32_t *topk_idx,
                         const int32_t *slot_pos, void *send,
                         hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->T == 0) return MOE_OK;
  if (!node_send || !node_slot || !topk_idx || !slot_pos || !send)
    return MOE_EINVAL;
  if (!aligned16(node_send) || !aligned16(send)) return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_forward(*cfg, node_send, node_slot,
                                           topk_idx, slot_pos, send, stream));
}

int moe_combine_partial(const moe_cfg *cfg, const void *y,
                        const int32_t *slot_pos, const float *topk_w,
                        const int32_t *topk_idx, const float *expert_scale,
                        const int32_t *node_slot, int32_t part_dtype,
                        void *part, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (part_dtype != MOE_F32 && part_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!y || !slot_pos || !topk_w || !topk_idx || !node_slot || !part)
    return MOE_EINVAL;
  if (!aligned16(y) || !aligned16(part)) return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_partial(*cfg, y, slot_pos, topk_w,
                                           topk_idx, expert_scale, node_slot,
                                           part_dtype, part, stream));
}

int moe_combine_nodes(const moe_cfg *cfg, const void *part,
                      int32_t part_dtype, const int32_t *node_slot, void *out,
                      hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (part_dtype != MOE_F32 && part_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!part || !node_slot || !out) return MOE_EINVAL;
  if (!aligned16(part) || !aligned16(out)) return MOE_EUNSUPPORTED;
  return launch_status(
      moe::launch_sum_nodes(*cfg, part, part_dtype, node_slot, out, stream));
}

int moe_dispatch_combine_nodes(const moe_cfg *cfg, const void *x,
                               const float *logits, const float *expert_scale,
                               int32_t *topk_idx, float *topk_w,
                               const moe_layout *layout, void *node_send,
                               void *send, int32_t part_dtype, void *part,
                               void *out, void *ws, size_t ws_bytes,
                               hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (part_dtype != MOE_F32 && part_dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if ((rc = check_layout_ptrs(cfg, layout)) != MOE_OK) return rc;
  if ((rc = check_ws(cfg, ws, ws_bytes)) != MOE_OK) return rc;
  if (cfg->T > 0) {
    if (!x || !logits || !topk_idx || !topk_w || !node_send || !send ||
        !part || !out || !layout->node_slot)
      return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(node_send) || !aligned16(send) ||
        !aligned16(part) || !aligned16(out))
      return MOE_EUNSUPPORTED;
  }
  const moe_layout &l = *layout;
  hipError_t e = moe::launch_gate(*cfg, logits, topk_idx, topk_w, stream);
  if (e == hipSuccess) e = moe::launch_layout(*cfg, topk_idx, l, ws, stream);
  if (e == hipSuccess)
    e = moe::launch_pack_nodes(*cfg, x, l.node_slot, node_send, stream);
  if (e == hipSuccess)
    e = moe::launch_forward(*cfg, node_send, l.node_slot, topk_idx,
                            l.slot_pos, send, stream);
  if (e == hipSuccess)
    e = moe::launch_partial(*cfg, send, l.slot_pos, topk_w, topk_idx,
                            expert_scale, l.node_slot, part_dtype, part,
                            stream);
  if (e == hipSuccess)
    e = moe::launch_sum_nodes(*cfg, part, part_dtype, l.node_slot, out,
                              stream);
  return launch_status(e);
}

size_t moe_fp8_row_bytes(int32_t H, int32_t qblock) {
  if (H < 1 || (qblock != 32 && qblock != 64 && qblock != 128) ||
      H % qblock != 0 || H % 16 != 0)
    return 0;
  return moe::fp8_row_bytes(H, qblock);
}

int moe_dispatch_pack_fp8(const moe_cfg *cfg, const void *x,
                          const int32_t *slot_pos, int32_t qblock, void *send,
                          hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (!moe::fp8_block_ok(*cfg, qblock)) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!x || !slot_pos || !send) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(send) || !aligned(slot_pos, 4))
    return MOE_EUNSUPPORTED;
  return launch_status(
      moe::launch_pack_fp8(*cfg, qblock, x, slot_pos, send, stream));
}

int moe_combine_fp8(const moe_cfg *cfg, const void *y, int32_t qblock,
                    const int32_t *slot_pos, const float *topk_w,
                    const int32_t *topk_idx, const float *expert_scale,
                    void *out, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (!moe::fp8_block_ok(*cfg, qblock)) return MOE_EUNSUPPORTED;
  if (cfg->T == 0) return MOE_OK;
  if (!y || !slot_pos || !topk_w || !out) return MOE_EINVAL;
  if (expert_scale && !topk_idx) return MOE_EINVAL;
  if (!aligned16(y) || !aligned16(out)) return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_combine_fp8(*cfg, qblock, y, slot_pos,
                                               topk_w, topk_idx, expert_scale,
                                               out, stream));
}

int moe_dispatch_combine_fp8(const moe_cfg *cfg, const void *x,
                             const float *logits, const float *expert_scale,
                             int32_t *topk_idx, float *topk_w,
                             const moe_layout *layout, int32_t qblock,
                             void *send, void *out, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (!moe::fp8_block_ok(*cfg, qblock)) return MOE_EUNSUPPORTED;
  if ((rc = check_layout_ptrs(cfg, layout)) != MOE_OK) return rc;
  if ((rc = check_ws(cfg, ws, ws_bytes)) != MOE_OK) return rc;
  if (cfg->T > 0) {
    if (!x || !logits || !topk_idx || !topk_w || !send || !out)
      return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(send) || !aligned16(out))
      return MOE_EUNSUPPORTED;
  }
  hipError_t e = moe::launch_gate(*cfg, logits, topk_idx, topk_w, stream);
  if (e == hipSuccess) e = moe::launch_layout(*cfg, topk_idx, *layout, ws, stream);
  if (e == hipSuccess)
    e = moe::launch_pack_fp8(*cfg, qblock, x, layout->slot_pos, send, stream);
  if (e == hipSuccess)
    e = moe::launch_combine_fp8(*cfg, qblock, send, layout->slot_pos, topk_w,
                                topk_idx, expert_scale, out, stream);
  return launch_status(e);
}

size_t moe_capacity_workspace_bytes(const moe_cfg *cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return moe::capacity_ws_bytes(*cfg);
}

static int check_cap_layout(const moe_cfg *c, const moe_capacity_layout *l) {
  if (!l || !l->expert_count || !l->expert_cap || !l->expert_off ||
      !l->row_src || !l->dropped)
    return MOE_EINVAL;
  if (c->T > 0 && !l->slot_pos) return MOE_EINVAL;
  return MOE_OK;
}

int moe_dispatch_layout_capacity(const moe_cfg *cfg, const int32_t *topk_idx,
                                 const int32_t *levels, int32_t q,
                                 const moe_capacity_layout *layout, void *ws,
                                 size_t ws_bytes, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (!moe::levels_ok(*cfg, levels, q)) return MOE_EINVAL;
  if ((rc = check_cap_layout(cfg, layout)) != MOE_OK) return rc;
  if (cfg->T > 0 && !topk_idx) return MOE_EINVAL;
  if (!ws) return MOE_EWORKSPACE;
  if (!aligned(ws, 256)) return MOE_EUNSUPPORTED;
  if (ws_bytes < moe::capacity_ws_bytes(*cfg)) return MOE_EWORKSPACE;
  return launch_status(moe::launch_layout_capacity(*cfg, topk_idx, levels, q,
                                                   *layout, ws, stream));
}

int moe_dispatch_pack_capacity(const moe_cfg *cfg, const void *x,
                               const int32_t *slot_pos,
                               const int32_t *row_src, int32_t n_rows,
                               void *send, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (n_rows < 0) return MOE_EINVAL;
  if (n_rows == 0 && cfg->T == 0) return MOE_OK;
  if (!send || !row_src || (cfg->T > 0 && (!x || !slot_pos)))
    return MOE_EINVAL;
  if ((x && !aligned16(x)) || !aligned16(send)) return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_pack_capacity(*cfg, x, slot_pos, row_src,
                                                 n_rows, send, stream));
}

int moe_combine_capacity(const moe_cfg *cfg, const void *y, int32_t n_rows,
                         const int32_t *slot_pos, const float *topk_w,
                         const int32_t *topk_idx, const float *expert_scale,
                         void *out, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (n_rows < 0) return MOE_EINVAL;
  if (cfg->T == 0) return MOE_OK;
  if (!y || !slot_pos || !topk_w || !out) return MOE_EINVAL;
  if (expert_scale && !topk_idx) return MOE_EINVAL;
  if (!aligned16(y) || !aligned16(out)) return MOE_EUNSUPPORTED;
  return launch_status(moe::launch_combine(*cfg, y, slot_pos, topk_w,
                                           topk_idx, expert_scale, out,
                                           stream, n_rows));
}

int moe_dispatch_combine_capacity(const moe_cfg *cfg, const void *x,
                                  const float *logits,
                                  const float *expert_scale,
                                  int32_t *topk_idx, float *topk_w,
                                  const int32_t *levels, int32_t q,
                                  const moe_capacity_layout *layout,
                                  void *send, void *out, void *ws,
                                  size_t ws_bytes, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (!moe::levels_ok(*cfg, levels, q)) return MOE_EINVAL;
  if ((rc = check_cap_layout(cfg, layout)) != MOE_OK) return rc;
  if (!ws) return MOE_EWORKSPACE;
  if (!aligned(ws, 256)) return MOE_EUNSUPPORTED;
  if (ws_bytes < moe::capacity_ws_bytes(*cfg)) return MOE_EWORKSPACE;
  if (!send) return MOE_EINVAL;
  if (cfg->T > 0) {
    if (!x || !logits || !topk_idx || !topk_w || !out) return MOE_EINVAL;
    if (!aligned16(x) || !aligned16(out)) return MOE_EUNSUPPORTED;
  }
  if (!aligned16(send)) return MOE_EUNSUPPORTED;
  const int n_rows = cfg->E * levels[q - 1];
  hipError_t e = moe::launch_gate(*cfg, logits, topk_idx, topk_w, stream);
  if (e == hipSuccess)
    e = moe::launch_layout_capacity(*cfg, topk_idx, levels, q, *layout, ws,
                                    stream);
  if (e == hipSuccess)
    e = moe::launch_pack_capacity(*cfg, x, layout->slot_pos, layout->row_src,
                                  n_rows, send, stream);
  if (e == hipSuccess)
    e = moe::launch_combine(*cfg, send, layout->slot_pos, topk_w, topk_idx,
                            expert_scale, out, stream, n_rows);
  return launch_status(e);
}

size_t moe_assign_workspace_bytes(const moe_cfg *cfg) {
  if (validate(cfg) != MOE_OK || !moe::assign_ok(*cfg)) return 0;
  return moe::assign_ws_bytes(*cfg);
}

int moe_assign_tasks(const moe_cfg *cfg, const int32_t *topk_idx,
                     const int32_t *src_rank, const uint8_t *holds,
                     const uint32_t *u_node, const uint32_t *u_rank,
                     int32_t *assign_rank, uint64_t *remote_mask, void *ws,
                     size_t ws_bytes, hipStream_t stream) {
  int rc = validate(cfg);
  if (rc != MOE_OK) return rc;
  if (!moe::assign_ok(*cfg)) return MOE_EUNSUPPORTED;
  if (!holds) return MOE_EINVAL;
  if (cfg->T > 0 && (!topk_idx || !src_rank || !u_node || !u_rank ||
                     !assign_rank || !remote_mask))
    return MOE_EINVAL;
  if (remote_mask && !aligned(remote_mask, 8)) return MOE_EUNSUPPORTED;
  if (!ws) return MOE_EWORKSPACE;
  if (!aligned(ws, 256)) return MOE_EUNSUPPORTED;
  if (ws_bytes < moe::assign_ws_bytes(*cfg)) return MOE_EWORKSPACE;
  return launch_status(moe::launch_assign(*cfg, topk_idx, src_rank, holds,
                                          u_node, u_rank, assign_rank,
                                          remote_mask, ws, stream));
}

int moe_read_device_error(const void *ws, hipStream_t stream,
                          int32_t *host_code, int clear) {
  if (!ws || !host_code) return MOE_EINVAL;
  int32_t v = 0;
  if (hipMemcpyAsync(&v, ws, sizeof v, hipMemcpyDeviceToHost, stream) !=
      hipSuccess)
    return MOE_ELAUNCH;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ELAUNCH;
  *host_code = v;
  if (clear) {
    if (moe::launch_fill_u32((uint32_t *)ws, 0u, 1, stream) != hipSuccess)
      return MOE_ELAUNCH;
  }
  return MOE_OK;
}

const char *moe_strerror(int code) {
  switch (code) {
    case MOE_OK: return "success";
    case MOE_EINVAL: return "invalid argument or inconsistent shape";
    case MOE_EUNSUPPORTED: return "unsupported dtype, alignment or size";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_ELAUNCH: return "HIP launch or copy failed";
    case MOE_ESCRATCH:
      return "workspace larger than the library's static scratch (1 MiB)";
    default: return "unknown error code";
  }
}

int moe_version(void) { return kVersion; }

}  // extern "C"
