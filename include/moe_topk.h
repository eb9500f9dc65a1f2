/*
 * moe_topk.h -- C ABI of the MI355X (gfx950) MoE dispatch/combine library.
 *
 * One GPU's share of Mixture-of-Experts token dispatch and combine, as four
 * stream-ordered steps plus their composition:
 *
 *   moe_topk_gate        top-K experts per token and their gate weights
 *   moe_dispatch_layout  counts, offsets, node-level dedup and the dispatch
 *                        permutation
 *   moe_dispatch_pack    hidden rows copied into contiguous per-rank,
 *                        expert-major send buffers
 *   moe_combine          expert rows gathered back to token order and summed
 *                        with the gate weights
 *   moe_dispatch_combine all four in order, the combine reading the packed
 *                        rows back through a diagonal stand-in expert
 *
 * The problem statement these calls follow is the one in "Efficient and
 * portable mixture-of-experts communication" (sections "Introdución",
 * "Envío (Dispatch)" and "Combinación (Combine)"): dispatch consumes tokens plus routing and emits
 * contiguous per-expert row buffers and per-token routing metadata; combine
 * consumes expert rows, that metadata and the weights, and writes an
 * externally allocated output; buffers are sized for the worst case; and no
 * step needs a GPU-to-host round trip for counts.
 *
 * Notation: T tokens, H hidden size, E experts, K experts per token, R
 * logical expert-parallel ranks holding E/R contiguous experts each, N
 * logical nodes holding R/N contiguous ranks each.  Ranks and nodes are
 * partitions of one GPU's buffers; nothing here talks to another GPU.
 *
 * Conventions for every call:
 *  - All array arguments are DEVICE pointers to memory the caller owns
 *    (allocated with hipMalloc or a framework allocator).  The library keeps
 *    no pointer after a call returns, allocates nothing, and holds no
 *    mutable global state.
 *  - Every call validates its arguments on the host, enqueues its kernels on
 *    `stream` and returns immediately.  Results are valid once the stream
 *    reaches that point.  Nothing but moe_read_device_error synchronises.
 *  - Row buffers (x, send, y, out) must be 16-byte aligned; other arrays
 *    need their natural alignment.  Matrices are dense and row-major.
 *  - Return value: MOE_OK, or a negative MOE_E* code; on error nothing is
 *    enqueued (MOE_ELAUNCH: a launch failed after earlier ones of the same
 *    call may have been enqueued).  Nothing throws across this ABI.
 *  - Inputs never hold NaN; results for NaN logits or rows are unspecified.
 */
#ifndef MOE_TOPK_H
#define MOE_TOPK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ------------------------------------------------------ */
#define MOE_OK 0
#define MOE_EINVAL (-1)       /* null required pointer or inconsistent shape */
#define MOE_EUNSUPPORTED (-2) /* valid but not supported: dtype, alignment   */
#define MOE_EWORKSPACE (-3)   /* workspace missing or smaller than required  */
#define MOE_ELAUNCH (-4)      /* a HIP launch or copy reported an error      */
#define MOE_ESCRATCH (-5)     /* needs more than the library's static scratch */

/* ---- device-detected input errors (bits of the workspace error word) --- */
#define MOE_DEVERR_EXPERT_RANGE 0x1 /* a topk_idx entry outside [0, E)      */
#define MOE_DEVERR_DUP_EXPERT 0x2   /* one token lists an expert twice      */
#define MOE_DEVERR_NO_REPLICA 0x4   /* an expert with no replica anywhere   */
#define MOE_DEVERR_SRC_RANK 0x8     /* a source rank outside [0, R)         */

/* ---- element types ----------------------------------------------------- */
#define MOE_F32 0  /* IEEE binary32                                         */
#define MOE_BF16 1 /* bfloat16 (upper half of binary32), ties-to-even       */

/* ---- flags ------------------------------------------------------------- */
/* Gate weights are the softmax over all E experts evaluated at the chosen
 * ones, instead of the default softmax over the K chosen (which sums to 1). */
#define MOE_F_NO_RENORM 0x1u

/* Problem description shared by all calls. */
typedef struct moe_cfg {
  int32_t T;           /* tokens, 0..2^31 - 4097; T * K < 2^31              */
  int32_t H;           /* hidden size, >= 1, multiple of 8                    */
  int32_t E;           /* experts, 1..4096                                    */
  int32_t K;           /* experts per token, 1..min(E, 32)                    */
  int32_t R;           /* logical ranks, E % R == 0; rank(e) = e / (E/R)      */
  int32_t N;           /* logical nodes, R % N == 0, N <= 64;
                          node(r) = r / (R/N)                                 */
  int32_t x_dtype;     /* MOE_F32 or MOE_BF16: x, send and y rows             */
  int32_t out_dtype;   /* MOE_F32 or MOE_BF16: combine output                 */
  uint32_t flags;      /* MOE_F_* bits                                        */
  int32_t layout_tile; /* tokens per layout workgroup: 64, 128, 256, 512 or
                          1024, or 0 for the default: 256 when T <= 256,
                          else 256 halved (down to 64) while that leaves
                          fewer than 91 tiles and a table of at most 256 KiB
                          ((tiles + 1) * (E + R + N) int32).  Results do not
                          depend on it; the workspace size does.              */
} moe_cfg;

/* Outputs of the dispatch layout (device pointers, caller-allocated).
 * Required: expert_count, expert_off, rank_count, rank_off, slot_pos,
 * row_src.  Optional (NULL skips the output): rank_token_count, node_mask,
 * node_count, node_off, node_slot. */
typedef struct moe_layout {
  int32_t *expert_count;     /* [E]   rows bound for expert e                  */
  int32_t *expert_off;       /* [E+1] exclusive prefix sum of expert_count     */
  int32_t *rank_count;       /* [R]   rows bound for rank r                    */
  int32_t *rank_off;         /* [R+1] first send row of rank r                 */
  int32_t *rank_token_count; /* [R]   distinct tokens with an expert on r      */
  uint64_t *node_mask;       /* [T]   bit n: token has an expert on node n     */
  int32_t *node_count;       /* [N]   tokens crossing to node n (once each)    */
  int32_t *node_off;         /* [N+1] exclusive prefix sum of node_count       */
  int32_t *node_slot;        /* [T*N] position of (t,n) in the node-major,
                                token-ascending list of crossings, or -1      */
  int32_t *slot_pos;         /* [T*K] send row of (t,k)                        */
  int32_t *row_src;          /* [T*K] inverse: row_src[slot_pos[i]] == i       */
} moe_layout;

/* Host-only check of a configuration; touches no device.  Returns MOE_OK,
 * MOE_EINVAL (bad shape) or MOE_EUNSUPPORTED (dtype, H alignment). */
int moe_validate_cfg(const moe_cfg *cfg);

/* Bytes of device workspace moe_dispatch_layout and moe_dispatch_combine
 * need for `cfg` (a 256-byte header holding the device error word, then
 * per-workgroup count tables).  0 when cfg is invalid.  Host only. */
size_t moe_workspace_bytes(const moe_cfg *cfg);

/* Clear the workspace header (the device error word).  Call once after
 * allocating a workspace; the workspace can then be reused by any number of
 * calls on the same stream.  Enqueued on `stream`. */
int moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Top-K gate ("Efficient and portable mixture-of-experts communication",
 * "Introdución": a router distribution over experts, the top-K scoring
 * experts, a weighted average with weights from that distribution).
 *   logits   [T*E] fp32 router scores, row-major by token.
 *   topk_idx [T*K] int32 out: the K experts with the largest logits, in
 *            descending logit order; equal logits go to the lower expert
 *            index (-0.0 equals +0.0).
 *   topk_w   [T*K] fp32 out: exp(l_k - l_max) / sum_j exp(l_j - l_max) over
 *            the K chosen (MOE_F_NO_RENORM: over all E), computed in fp64
 *            and rounded once to fp32. */
int moe_topk_gate(const moe_cfg *cfg, const float *logits, int32_t *topk_idx,
                  float *topk_w, hipStream_t stream);

/* Dispatch layout (same page, "Envío (Dispatch)": per-destination token counts and
 * contiguous per-expert buffers with (rank, expert, token) kept for the
 * combine; "Workload-Static Optical Circuit Switching for Scalable LLM
 * Inference Decode", "Variable MoE Traffic and Regularization": rows per
 * destination group, worst-case buffers; "Cobalt: Leveraging Expert
 * Co-activation for Efficient Distributed MoE Training", Section 1: a token
 * crosses to a node once however many of its experts live there).
 *   topk_idx [T*K] int32 expert ids; each row must list K distinct ids in
 *            [0, E).  Violations set MOE_DEVERR_* bits in the workspace
 *            error word; outputs are then unspecified but every write stays
 *            in bounds (slot_pos entries of bad ids are -1).
 *   layout   outputs, see moe_layout.  The send row order is expert-major
 *            (expert 0's rows first) and, inside an expert, token-ascending;
 *            rank r's rows are [rank_off[r], rank_off[r+1]).
 *   ws       workspace of at least moe_workspace_bytes(cfg) bytes,
 *            initialised once with moe_workspace_init. */
int moe_dispatch_layout(const moe_cfg *cfg, const int32_t *topk_idx,
                        const moe_layout *layout, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* Dispatch pack ("Efficient and portable mixture-of-experts communication",
 * "Envío (Dispatch)": token rows are packed into contiguous chunks per destination).
 *   x        [T*H] rows of x_dtype.
 *   slot_pos [T*K] send row of each (t,k), e.g. from moe_dispatch_layout.
 *   send     [T*K*H] out, x_dtype: send[slot_pos[t*K+k]] = x[t], bit for
 *            bit.  Rows no slot names are left untouched.  A slot outside
 *            [0, T*K) is skipped. */
int moe_dispatch_pack(const moe_cfg *cfg, const void *x,
                      const int32_t *slot_pos, void *send,
                      hipStream_t stream);

/* Combine (same page, "Combinación (Combine)": the receiver reads the K expert rows of
 * each token and forms their weighted average into an externally allocated
 * output; "Fragmentación e paralelismo": the accumulation is fused into the
 * gather).
 *   y            [T*K*H] expert output rows of x_dtype, in send-row order.
 *   slot_pos     [T*K] row of y holding (t,k); rows outside [0, T*K) add 0.
 *   topk_w       [T*K] fp32 gate weights.
 *   topk_idx     [T*K] int32 expert ids; read only when expert_scale is set.
 *   expert_scale [E] fp32 or NULL: per-expert factor s_e applied to expert
 *                e's rows (a diagonal stand-in expert); NULL means s = 1.
 *   out          [T*H] out_dtype: sum_k w[t,k]*s[e(t,k)]*y[slot_pos[t,k]],
 *                accumulated in fp32, rounded to nearest-even once. */
int moe_combine(const moe_cfg *cfg, const void *y, const int32_t *slot_pos,
                const float *topk_w, const int32_t *topk_idx,
                const float *expert_scale, void *out, hipStream_t stream);

/* The whole path on one GPU: gate -> layout -> pack -> combine, where the
 * combine reads the packed rows back from `send` (on one GPU a rank's
 * receive buffer is its own segment of send) through the diagonal stand-in
 * expert s_e.  out is computed from send, never from x directly.  Outputs:
 * topk_idx, topk_w, layout, send and out, each as in the calls above. */
int moe_dispatch_combine(const moe_cfg *cfg, const void *x,
                         const float *logits, const float *expert_scale,
                         int32_t *topk_idx, float *topk_w,
                         const moe_layout *layout, void *send, void *out,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_dispatch_combine without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The layout's workspace
 * (error word and per-tile count table, moe_workspace_bytes(cfg) bytes) is
 * kept in a static device array of MOE_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends; the call allocates
 * nothing.  The caller passes every input and output, as above, and gets the
 * same results.  Returns MOE_ESCRATCH, before anything is enqueued, when
 * moe_workspace_bytes(cfg) exceeds MOE_SCRATCH_BYTES (1 MiB, with the
 * default layout tile: up to 204288 tokens at E = 256, R = 64, N = 8;
 * 64256 at E = 896, R = 128, N = 16; 3904 at E = 4096).
 * `stream` must belong to the current device.  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race, so the caller orders them.  The array's error word is
 * cleared at the start of each call; the expert ids come from the call's
 * own gate, so no device-detected error arises. */
#define MOE_SCRATCH_BYTES (1u << 20)
int moe_dispatch_combine_noalloc(const moe_cfg *cfg, const void *x,
                                 const float *logits,
                                 const float *expert_scale, int32_t *topk_idx,
                                 float *topk_w, const moe_layout *layout,
                                 void *send, void *out, hipStream_t stream);

/* ---- node-level two-leg dispatch and hierarchical combine -------------
 * "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
 * Training", Section 1: a token whose experts share a node crosses to that
 * node once and is forwarded inside it.  "MoX: Efficient MoE Routing on
 * Direct-Connect Topologies", Section 2.5: on the way back a node reduces
 * the expert outputs it holds for a token and forwards one vector.
 * The leg-1 buffer node_send and the partial buffer part have
 * moe_node_rows_max(cfg) = T * min(K, N) rows of H elements; the rows in
 * use are [0, node_off[N]), node-major with tokens ascending (node_slot from
 * moe_dispatch_layout).  node(e) = (e / (E/R)) / (R/N). */

/* Rows of the node_send and part buffers for cfg (0 when cfg is invalid).
 * Host only. */
size_t moe_node_rows_max(const moe_cfg *cfg);

/* Leg 1: node_send[node_slot[t*N+n]] = x[t] (x_dtype rows, bit for bit)
 * for every (t, n) with node_slot >= 0.  node_slot [T*N] int32 as produced
 * by moe_dispatch_layout; entries outside [0, moe_node_rows_max) skipped. */
int moe_dispatch_pack_nodes(const moe_cfg *cfg, const void *x,
                            const int32_t *node_slot, void *node_send,
                            hipStream_t stream);

/* Leg 2: send[slot_pos[t*K+k]] = node_send[node_slot[t*N + node(e)]] with
 * e = topk_idx[t*K+k]: the row that reached expert e's node is forwarded to
 * the expert's segment.  With node_send from moe_dispatch_pack_nodes, send
 * equals what moe_dispatch_pack writes.  Slots with an expert id outside
 * [0, E), a send row outside [0, T*K) or no node row are skipped. */
int moe_dispatch_forward(const moe_cfg *cfg, const void *node_send,
                         const int32_t *node_slot, const int32_t *topk_idx,
                         const int32_t *slot_pos, void *send,
                         hipStream_t stream);

/* Reverse of leg 2, per node: for every (t, n) with node_slot >= 0,
 *   part[node_slot[t*N+n]] = sum over k with node(e(t,k)) == n of
 *                            w[t,k] * s[e(t,k)] * y[slot_pos[t,k]]
 * accumulated in fp32 and rounded to nearest-even once into part_dtype
 * (MOE_F32 or MOE_BF16).  y, slot_pos, topk_w, expert_scale as in
 * moe_combine; topk_idx is required (it places each slot on a node). */
int moe_combine_partial(const moe_cfg *cfg, const void *y,
                        const int32_t *slot_pos, const float *topk_w,
                        const int32_t *topk_idx, const float *expert_scale,
                        const int32_t *node_slot, int32_t part_dtype,
                        void *part, hipStream_t stream);

/* Reverse of leg 1, at the source: out[t] = sum over n with node_slot >= 0
 * of part[node_slot[t*N+n]], accumulated in fp32 and rounded once into
 * out_dtype. */
int moe_combine_nodes(const moe_cfg *cfg, const void *part,
                      int32_t part_dtype, const int32_t *node_slot, void *out,
                      hipStream_t stream);

/* The two-leg path: gate -> layout (layout->node_slot required) -> leg 1 ->
 * leg 2 -> per-node partials of the stand-in expert applied to send ->
 * sum at the source.  Outputs as in the calls above; out is computed from
 * the partials, never from x. */
int moe_dispatch_combine_nodes(const moe_cfg *cfg, const void *x,
                               const float *logits, const float *expert_scale,
                               int32_t *topk_idx, float *topk_w,
                               const moe_layout *layout, void *node_send,
                               void *send, int32_t part_dtype, void *part,
                               void *out, void *ws, size_t ws_bytes,
                               hipStream_t stream);

/* ---- FP8 dispatch with per-block scales ---------------------------------
 * "Efficient and portable mixture-of-experts communication", "Envío
 * (Dispatch)": tokens travel with block scale factors; "Workload-Static
 * Optical Circuit Switching for Scalable LLM Inference Decode",
 * "Communication precision": FP8 transport for MoE dispatch.  Format of a
 * packed row (qblock B in {32, 64, 128}, H % B == 0, H % 16 == 0, and a row
 * tail of scales and padding of at most 16 KiB, about H/B <= 4064; other
 * shapes give MOE_EUNSUPPORTED):
 *   bytes [0, H)            OCP E4M3 codes (bias 7, largest magnitude 448,
 *                           round to nearest even, sign kept)
 *   bytes [H, H + 4H/B)     one fp32 scale per block of B elements
 *   bytes up to the stride  zero padding; stride = moe_fp8_row_bytes(H, B),
 *                           a multiple of 128 (no 128-byte block holds
 *                           parts of two rows)
 * For a block with largest magnitude amax: scale = amax / 448 and
 * code_i = e4m3(min(max(x_i * (448 / amax), -448), 448)), each operation in
 * fp32 with round to nearest even; a block of zeros has scale 0 and zero
 * codes.  The dequantised value is value(code) * scale. */

/* Row stride in bytes of a packed FP8 row, or 0 for an unsupported
 * (H, qblock).  Host only. */
size_t moe_fp8_row_bytes(int32_t H, int32_t qblock);

/* Quantising pack: each token's row of x is quantised once and written to
 * its K send rows, send + slot_pos[t*K+k] * moe_fp8_row_bytes(H, qblock).
 * send holds T*K rows; rows no slot names are left untouched; a slot
 * outside [0, T*K) is skipped. */
int moe_dispatch_pack_fp8(const moe_cfg *cfg, const void *x,
                          const int32_t *slot_pos, int32_t qblock, void *send,
                          hipStream_t stream);

/* Combine of FP8 rows: out[t] = sum_k w[t,k] * s[e(t,k)] * deq(y[slot_pos[t,k]])
 * accumulated in fp32 and rounded once into out_dtype; other arguments as
 * in moe_combine. */
int moe_combine_fp8(const moe_cfg *cfg, const void *y, int32_t qblock,
                    const int32_t *slot_pos, const float *topk_w,
                    const int32_t *topk_idx, const float *expert_scale,
                    void *out, hipStream_t stream);

/* gate -> layout -> quantising pack -> combine of the FP8 rows through the
 * diagonal stand-in expert.  out is computed from send, never from x. */
int moe_dispatch_combine_fp8(const moe_cfg *cfg, const void *x,
                             const float *logits, const float *expert_scale,
                             int32_t *topk_idx, float *topk_w,
                             const moe_layout *layout, int32_t qblock,
                             void *send, void *out, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* ---- capacity-padded and bucketed layout -------------------------------
 * "Workload-Static Optical Circuit Switching for Scalable LLM Inference
 * Decode", "Variable MoE Traffic and Regularization": every buffer between a
 * source and a destination expert is padded to a fixed capacity, so each
 * step moves the same volume, and rows beyond it are dropped; bucketing
 * rounds each count up to one of q levels C_1 < ... < C_q.  The page's
 * capacity formula is missing; C = ceil(gamma * T * K / E) is the intended
 * use (levels = {C}).  With Cmax = levels[q-1]:
 *   kept_e  = min(expert_count[e], Cmax): expert e keeps its first kept_e
 *             tokens in token order, the rest are dropped;
 *   expert_cap[e] = smallest level >= kept_e; expert_off = exclusive prefix;
 *   slot_pos[t*K+k] = expert_off[e] + rank of t among e's tokens, or -1;
 *   row_src[r] = t*K + k for used rows, -1 for padding rows
 *                (E * Cmax entries, the capacity of a send buffer);
 *   *dropped = sum_e (expert_count[e] - kept_e).
 * A dropped (t, k) adds nothing in the combine; the other weights are not
 * rescaled. */
#define MOE_MAX_LEVELS 8

typedef struct moe_capacity_layout {
  int32_t *expert_count; /* [E]   times expert e was chosen               */
  int32_t *expert_cap;   /* [E]   rows of expert e's padded segment       */
  int32_t *expert_off;   /* [E+1] first row of each segment              */
  int32_t *slot_pos;     /* [T*K] send row of (t,k), -1 when dropped      */
  int32_t *row_src;      /* [E*Cmax] t*K+k of a used row, -1 for padding  */
  int32_t *dropped;      /* [1]   number of dropped (t,k)                 */
} moe_capacity_layout;

/* Workspace bytes moe_dispatch_layout_capacity and
 * moe_dispatch_combine_capacity need (0 when cfg is invalid).  Host only. */
size_t moe_capacity_workspace_bytes(const moe_cfg *cfg);

/* Capacity-padded / bucketed layout of topk_idx.  levels is a HOST array of
 * q (1..MOE_MAX_LEVELS) strictly increasing positive row counts; every
 * output pointer of `layout` is required. */
int moe_dispatch_layout_capacity(const moe_cfg *cfg, const int32_t *topk_idx,
                                 const int32_t *levels, int32_t q,
                                 const moe_capacity_layout *layout, void *ws,
                                 size_t ws_bytes, hipStream_t stream);

/* Pack into a padded send buffer of n_rows rows: used rows receive their
 * token's x row, rows with row_src < 0 are set to zero.  row_src must hold
 * n_rows entries (n_rows <= E * Cmax for the layout's row_src). */
int moe_dispatch_pack_capacity(const moe_cfg *cfg, const void *x,
                               const int32_t *slot_pos,
                               const int32_t *row_src, int32_t n_rows,
                               void *send, hipStream_t stream);

/* moe_combine over a padded buffer y of n_rows rows; slots outside
 * [0, n_rows) (dropped ones are -1) add nothing. */
int moe_combine_capacity(const moe_cfg *cfg, const void *y, int32_t n_rows,
                         const int32_t *slot_pos, const float *topk_w,
                         const int32_t *topk_idx, const float *expert_scale,
                         void *out, hipStream_t stream);

/* gate -> capacity layout -> padded pack -> combine through the stand-in
 * expert; send has E * levels[q-1] rows.  out is computed from send. */
int moe_dispatch_combine_capacity(const moe_cfg *cfg, const void *x,
                                  const float *logits,
                                  const float *expert_scale,
                                  int32_t *topk_idx, float *topk_w,
                                  const int32_t *levels, int32_t q,
                                  const moe_capacity_layout *layout,
                                  void *send, void *out, void *ws,
                                  size_t ws_bytes, hipStream_t stream);

/* ---- communication-aware task assignment ------------------------------
 * "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
 * Training", Section 3.3.  The R ranks of cfg sit on N nodes, R/N contiguous
 * ranks a node; holds[r*E + e] != 0 when rank r holds a replica of expert e
 * (any number of replicas per expert).  For token t from source rank
 * src_rank[t] (node sn):
 *   - a selected expert with a replica on node sn runs on node sn;
 *   - for the others, remote_mask[t] = the smallest set of remote nodes that
 *     holds each of them (bit n = node n); among sets of equal size the one
 *     with the smallest mask value;
 *   - each such expert runs on node number floor(u_node * c / 2^32) (in
 *     ascending order) of the c nodes of remote_mask[t] holding it;
 *   - assign_rank[t*K+k] = rank number floor(u_rank * c / 2^32) of the c
 *     ranks of that node holding the expert (ascending).
 * u_node, u_rank: [T*K] uint32 draws supplied by the caller (uniform draws
 * give the random and uniform choices of the page).  An expert id outside
 * [0, E), an expert without replica or a source rank outside [0, R) sets
 * the matching MOE_DEVERR_* bit, and that token's ranks are -1.  Needs at
 * most 24 nodes and at most 64 ranks per node (MOE_EUNSUPPORTED otherwise,
 * returned on the host before anything is enqueued): the cover search tests
 * up to 2^(N-1) node subsets per token, the cost the page states, so N is
 * kept to the small expert-parallel degrees it assumes. */

/* Workspace bytes of moe_assign_tasks (0 when cfg is invalid or N > 24).
 * Host only. */
size_t moe_assign_workspace_bytes(const moe_cfg *cfg);

int moe_assign_tasks(const moe_cfg *cfg, const int32_t *topk_idx,
                     const int32_t *src_rank, const uint8_t *holds,
                     const uint32_t *u_node, const uint32_t *u_rank,
                     int32_t *assign_rank, uint64_t *remote_mask, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/* Copy the workspace error word (MOE_DEVERR_* bits, 0 when clean) to
 * *host_code after all work queued on `stream`; synchronises `stream`.  When
 * `clear` is non-zero the word is reset to 0 afterwards (enqueued). */
int moe_read_device_error(const void *ws, hipStream_t stream,
                          int32_t *host_code, int clear);

/* Static text for a MOE_* return code. */
const char *moe_strerror(int code);

/* Library version as major*10000 + minor*100 + patch. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TOPK_H */
