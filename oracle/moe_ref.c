/*
 * moe_ref.c -- CPU oracle for MoE top-K gating, dispatch layout, dispatch
 * packing and the gate-weighted combine.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, single-threaded
 * statement of what the path computes.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may build, load or call it.  It shares no
 * code, header, table or helper with the HIP library, and includes nothing
 * from it.  Floating point that produces a value is done in fp64; fp32 is used
 * only where the inputs are fp32 (the logit comparisons that choose experts),
 * where a value is an integer decision taken in fp32 (FP8 codes), and in the
 * one function that states the fp32 value a stored 16-bit partial sum is
 * rounded from (moe_ref_combine_partial_f32).
 *
 * Sources (page title, section):
 *  - "Efficient and portable mixture-of-experts communication", "Introdución":
 *    a router produces a probability distribution over experts, the top-K
 *    scoring experts are chosen and the layer output is the weighted average
 *    of the chosen experts' outputs, weighted by values derived from that
 *    distribution.  Sections "Envío (Dispatch)" and "Combinación (Combine)": the sender counts the
 *    tokens bound for every destination expert and packs token rows into
 *    contiguous chunks; the receiver lays them out as contiguous per-expert
 *    buffers for a grouped GEMM and keeps (rank, expert, token) so the
 *    combine can find each row; the combine reads the K expert rows of a
 *    token and forms their weighted sum into an externally allocated output.
 *  - "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
 *    Training", Section 1: node-level deduplication -- a token crosses to a
 *    node once however many of its experts live there; Section 3.1: the
 *    task count sums to K*T.
 *  - "Workload-Static Optical Circuit Switching for Scalable LLM Inference
 *    Decode", section "Variable MoE Traffic and Regularization": the dispatch
 *    traffic entry W_uv counts the rows sent from group u to group v;
 *    production kernels size receive buffers for the worst case and drop
 *    nothing.
 *  - "MoX: Efficient MoE Routing on Direct-Connect Topologies", Section 2.1:
 *    a per-token destination bitmap, 8 bytes at 64 endpoints.
 *
 * Readings where the pages leave a step open (ties to the lower expert index;
 * selection by logit; softmax renormalised over the K chosen; experts placed
 * on ranks, and ranks on nodes, in contiguous blocks; one packed row per
 * (token, slot) in expert-major order with tokens ascending) are listed with
 * the design notes of the repository.
 *
 * Parity pins: every function below is checked in the CPU test-suite against
 * library routines (stable argsort, bincount, cumsum), closed forms and brute
 * force; none of them is "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define REF_OK 0
#define REF_EINVAL (-1)

#define REF_DT_F32 0
#define REF_DT_BF16 1

/* ------------------------------------------------------------------------ */
/* Scalar helpers                                                           */
/* ------------------------------------------------------------------------ */

/* Widen a bf16 bit pattern to its exact value. */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round an fp64 value to the nearest bf16 (ties to even) in one step and
 * return its bit pattern.  bf16 keeps 8 significant bits and the fp32
 * exponent range; below 2^-126 the spacing is fixed at 2^-133. */
uint16_t moe_ref_f64_to_bf16(double v) {
  double a = fabs(v);
  int neg = signbit(v) ? 1 : 0;
  double q;
  if (a == 0.0) {
    q = 0.0;
  } else {
    int ex;
    (void)frexp(a, &ex);          /* a = f * 2^ex, 0.5 <= f < 1 */
    int shift = 8 - ex;           /* a * 2^shift lies in [128, 256) */
    if (ex - 8 < -133) shift = 133; /* subnormal range: fixed quantum */
    q = ldexp(nearbyint(ldexp(a, shift)), -shift);
  }
  float f = (float)(neg ? -q : q); /* exact: q is a bf16 value */
  if (isinf(f) || fabs(q) >= ldexp(1.0, 128)) f = neg ? -INFINITY : INFINITY;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* "a ranks before b": larger logit first, equal logits by lower index.
 * -0.0 and +0.0 compare equal under IEEE comparison, which is the wanted
 * canonicalisation. */
static int ranks_before(float la, int ia, float lb, int ib) {
  if (la > lb) return 1;
  if (la < lb) return 0;
  return ia < ib;
}

/* ------------------------------------------------------------------------ */
/* 1. Gate                                                                   */
/* ------------------------------------------------------------------------ */

/* For every token t: choose the K experts that rank first under
 * (logit descending, expert index ascending), in that order, by K passes of
 * "take the best expert not yet taken".  Weights: softmax over the K chosen
 * (renorm != 0) or the full softmax over E evaluated at the chosen experts
 * (renorm == 0), in fp64 with the maximum subtracted, rounded once to fp32. */
int moe_ref_gate(int T, int E, int K, int renorm, const float *logits,
                 int32_t *topk_idx, float *topk_w) {
  if (T < 0 || E < 1 || K < 1 || K > E) return REF_EINVAL;
  unsigned char taken[8192];
  if (E > (int)sizeof taken) return REF_EINVAL;
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int k = 0; k < K; ++k) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      topk_idx[(size_t)t * K + k] = best;
    }
    double m = (double)l[topk_idx[(size_t)t * K]]; /* the largest logit */
    double denom = 0.0;
    if (renorm) {
      for (int k = 0; k < K; ++k)
        denom += exp((double)l[topk_idx[(size_t)t * K + k]] - m);
    } else {
      for (int e = 0; e < E; ++e) denom += exp((double)l[e] - m);
    }
    for (int k = 0; k < K; ++k) {
      double num = exp((double)l[topk_idx[(size_t)t * K + k]] - m);
      topk_w[(size_t)t * K + k] = (float)(num / denom);
    }
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* 2. Dispatch layout                                                        */
/* ------------------------------------------------------------------------ */

/* Experts sit on ranks in contiguous blocks of E/R, ranks on nodes in
 * contiguous blocks of R/N.  Outputs (any of rank_token_count, node_mask,
 * node_count, node_off, node_slot may be NULL):
 *   expert_count[E]   rows bound for expert e
 *   expert_off[E+1]   exclusive prefix sum of expert_count
 *   rank_count[R]     rows bound for rank r (one row of the traffic matrix)
 *   rank_off[R+1]     first row of rank r in the send buffer
 *   rank_token_count[R] distinct tokens with at least one expert on rank r
 *   node_mask[T]      bit n set when token t has an expert on node n
 *   node_count[N]     tokens whose mask has bit n (one crossing per node)
 *   node_off[N+1]     exclusive prefix sum of node_count
 *   node_slot[T*N]    position of (t, n) in the node-major, token-ascending
 *                     list of node crossings, or -1 when bit n is clear
 *   slot_pos[T*K]     row of (t, k) in the send buffer: rows are grouped by
 *                     expert in expert order; inside an expert, by (t, k)
 *   row_src[T*K]      inverse permutation: row_src[slot_pos[i]] = i
 * Returns REF_EINVAL for an expert id outside [0, E) or a bad shape. */
int moe_ref_layout(int T, int E, int K, int R, int N,
                   const int32_t *topk_idx, int32_t *expert_count,
                   int32_t *expert_off, int32_t *rank_count, int32_t *rank_off,
                   int32_t *rank_token_count, uint64_t *node_mask,
                   int32_t *node_count, int32_t *node_off, int32_t *node_slot,
                   int32_t *slot_pos, int32_t *row_src) {
  if (T < 0 || E < 1 || K < 1 || R < 1 || N < 1 || N > 64) return REF_EINVAL;
  if (E % R != 0 || R % N != 0) return REF_EINVAL;
  const int per_rank = E / R;
  const int per_node = R / N;
  const size_t TK = (size_t)T * K;

  for (size_t i = 0; i < TK; ++i)
    if (topk_idx[i] < 0 || topk_idx[i] >= E) return REF_EINVAL;

  /* (a) rows per expert and their exclusive scan */
  for (int e = 0; e < E; ++e) expert_count[e] = 0;
  for (size_t i = 0; i < TK; ++i) expert_count[topk_idx[i]] += 1;
  expert_off[0] = 0;
  for (int e = 0; e < E; ++e) expert_off[e + 1] = expert_off[e] + expert_count[e];

  /* (b) rows per rank: experts of rank r are [r*E/R, (r+1)*E/R) */
  for (int r = 0; r < R; ++r) {
    int32_t c = 0;
    for (int e = r * per_rank; e < (r + 1) * per_rank; ++e) c += expert_count[e];
    rank_count[r] = c;
  }
  rank_off[0] = 0;
  for (int r = 0; r < R; ++r) rank_off[r + 1] = rank_off[r] + rank_count[r];

  /* (c) distinct tokens per rank */
  if (rank_token_count) {
    for (int r = 0; r < R; ++r) rank_token_count[r] = 0;
    for (int t = 0; t < T; ++t) {
      for (int r = 0; r < R; ++r) {
        int hit = 0;
        for (int k = 0; k < K; ++k)
          if (topk_idx[(size_t)t * K + k] / per_rank == r) hit = 1;
        rank_token_count[r] += hit;
      }
    }
  }

  /* (d) node dedup: one crossing per (token, distinct node) */
  if (node_mask || node_count || node_off || node_slot) {
    int32_t cnt[64];
    int32_t seen[64];
    for (int n = 0; n < N; ++n) cnt[n] = 0;
    for (int t = 0; t < T; ++t) {
      uint64_t m = 0;
      for (int k = 0; k < K; ++k) {
        int node = (topk_idx[(size_t)t * K + k] / per_rank) / per_node;
        m |= (uint64_t)1 << node;
      }
      if (node_mask) node_mask[t] = m;
      for (int n = 0; n < N; ++n)
        if (m >> n & 1) cnt[n] += 1;
    }
    if (node_count)
      for (int n = 0; n < N; ++n) node_count[n] = cnt[n];
    int32_t off[65];
    off[0] = 0;
    for (int n = 0; n < N; ++n) off[n + 1] = off[n] + cnt[n];
    if (node_off)
      for (int n = 0; n <= N; ++n) node_off[n] = off[n];
    if (node_slot) {
      for (int n = 0; n < N; ++n) seen[n] = 0;
      for (int t = 0; t < T; ++t) {
        uint64_t m = 0;
        for (int k = 0; k < K; ++k) {
          int node = (topk_idx[(size_t)t * K + k] / per_rank) / per_node;
          m |= (uint64_t)1 << node;
        }
        for (int n = 0; n < N; ++n) {
          if (m >> n & 1) {
            node_slot[(size_t)t * N + n] = off[n] + seen[n];
            seen[n] += 1;
          } else {
            node_slot[(size_t)t * N + n] = -1;
          }
        }
      }
    }
  }

  /* (e) slot positions: walk (t, k) in order, each expert's rows fill its
   * segment from the front */
  for (int e = 0; e < E; ++e) expert_count[e] = 0; /* reuse as fill cursor */
  for (size_t i = 0; i < TK; ++i) {
    int e = topk_idx[i];
    slot_pos[i] = expert_off[e] + expert_count[e];
    expert_count[e] += 1;
  }
  /* expert_count is whole again: every cursor ended at its count */
  for (size_t i = 0; i < TK; ++i) row_src[slot_pos[i]] = (int32_t)i;
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* 3. Pack                                                                   */
/* ------------------------------------------------------------------------ */

/* send[slot_pos[t*K+k]] = x[t], copied byte for byte (row_bytes per row). */
int moe_ref_pack(int T, int K, size_t row_bytes, const void *x,
                 const int32_t *slot_pos, void *send) {
  if (T < 0 || K < 1) return REF_EINVAL;
  const unsigned char *src = (const unsigned char *)x;
  unsigned char *dst = (unsigned char *)send;
  for (int t = 0; t < T; ++t) {
    for (int k = 0; k < K; ++k) {
      int32_t s = slot_pos[(size_t)t * K + k];
      if (s < 0 || (size_t)s >= (size_t)T * K) return REF_EINVAL;
      memcpy(dst + (size_t)s * row_bytes, src + (size_t)t * row_bytes,
             row_bytes);
    }
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* 4. Combine                                                                */
/* ------------------------------------------------------------------------ */

/* out[t, h] = sum_k w[t,k] * s[e(t,k)] * y[slot_pos[t,k], h], summed in fp64
 * in k order; s = 1 when expert_scale is NULL (expert ids then unused).  A
 * negative slot (a slot dropped by a capacity-limited layout) adds nothing.
 * out_exact (may be NULL) receives the unrounded fp64 sum; out (may be NULL)
 * the sum rounded to nearest-even in out_dtype. */
int moe_ref_combine(int T, int H, int K, int y_dtype, const void *y,
                    const int32_t *slot_pos, const float *topk_w,
                    const int32_t *topk_idx, const float *expert_scale,
                    int out_dtype, void *out, double *out_exact) {
  if (T < 0 || H < 1 || K < 1) return REF_EINVAL;
  if (expert_scale && !topk_idx) return REF_EINVAL;
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        size_t i = (size_t)t * K + k;
        if (slot_pos[i] < 0) continue; /* dropped slot: contributes nothing */
        double c = (double)topk_w[i];
        if (expert_scale) c *= (double)expert_scale[topk_idx[i]];
        size_t at = (size_t)slot_pos[i] * H + h;
        double v = (y_dtype == REF_DT_F32) ? (double)((const float *)y)[at]
                                           : bf16_value(((const uint16_t *)y)[at]);
        acc += c * v;
      }
      size_t o = (size_t)t * H + h;
      if (out_exact) out_exact[o] = acc;
      if (out) {
        if (out_dtype == REF_DT_F32)
          ((float *)out)[o] = (float)acc;
        else
          ((uint16_t *)out)[o] = moe_ref_f64_to_bf16(acc);
      }
    }
  }
  return REF_OK;
}

/* Combine for a subset of tokens only (for sampled checks at full size):
 * tokens[j] names the token whose row j of out/out_exact is produced. */
int moe_ref_combine_tokens(int n_tokens, const int32_t *tokens, int H, int K,
                           int y_dtype, const void *y,
                           const int32_t *slot_pos, const float *topk_w,
                           const int32_t *topk_idx, const float *expert_scale,
                           double *out_exact) {
  if (n_tokens < 0 || H < 1 || K < 1) return REF_EINVAL;
  for (int j = 0; j < n_tokens; ++j) {
    int t = tokens[j];
    int r = moe_ref_combine(1, H, K, y_dtype,
                            y, slot_pos + (size_t)t * K, topk_w + (size_t)t * K,
                            topk_idx ? topk_idx + (size_t)t * K : NULL,
                            expert_scale, REF_DT_F32, NULL,
                            out_exact + (size_t)j * H);
    if (r != REF_OK) return r;
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* 5. Node-level two-leg dispatch and hierarchical combine                  */
/* ------------------------------------------------------------------------ */
/*
 * "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
 * Training", Section 1: when several of a token's experts live on one remote
 * node, the token crosses the inter-node link once and is forwarded inside
 * the node.  "MoX: Efficient MoE Routing on Direct-Connect Topologies",
 * Section 2.5: the combine runs the dispatch tree backwards and a node that
 * holds several of a token's expert outputs reduces them before forwarding
 * one vector toward the source.
 *
 * Leg 1 rows are node-major with tokens ascending inside a node: row
 * node_slot[t*N+n] (from moe_ref_layout) carries token t to node n.  D is
 * the number of such rows (the sum of node_count).
 */

/* Leg 1: node_send[node_slot[t*N+n]] = x[t] for every n with a slot >= 0. */
int moe_ref_pack_nodes(int T, int N, size_t row_bytes, const void *x,
                       const int32_t *node_slot, int D, void *node_send) {
  if (T < 0 || N < 1 || D < 0) return REF_EINVAL;
  const unsigned char *src = (const unsigned char *)x;
  unsigned char *dst = (unsigned char *)node_send;
  for (int t = 0; t < T; ++t) {
    for (int n = 0; n < N; ++n) {
      int32_t s = node_slot[(size_t)t * N + n];
      if (s < 0) continue;
      if (s >= D) return REF_EINVAL;
      memcpy(dst + (size_t)s * row_bytes, src + (size_t)t * row_bytes,
             row_bytes);
    }
  }
  return REF_OK;
}

/* Leg 2: the row that reached expert e's node is copied to the expert's
 * segment: send[slot_pos[t*K+k]] = node_send[node_slot[t*N + node(e)]] with
 * e = topk_idx[t*K+k], node(e) = (e / (E/R)) / (R/N). */
int moe_ref_forward(int T, int E, int K, int R, int N, size_t row_bytes,
                    const void *node_send, int D, const int32_t *node_slot,
                    const int32_t *topk_idx, const int32_t *slot_pos,
                    void *send) {
  if (T < 0 || E < 1 || K < 1 || R < 1 || N < 1) return REF_EINVAL;
  if (E % R != 0 || R % N != 0) return REF_EINVAL;
  const int per_rank = E / R, per_node = R / N;
  const unsigned char *src = (const unsigned char *)node_send;
  unsigned char *dst = (unsigned char *)send;
  for (int t = 0; t < T; ++t) {
    for (int k = 0; k < K; ++k) {
      size_t i = (size_t)t * K + k;
      int e = topk_idx[i];
      if (e < 0 || e >= E) return REF_EINVAL;
      int n = (e / per_rank) / per_node;
      int32_t from = node_slot[(size_t)t * N + n];
      int32_t to = slot_pos[i];
      if (from < 0 || from >= D || to < 0 || (size_t)to >= (size_t)T * K)
        return REF_EINVAL;
      memcpy(dst + (size_t)to * row_bytes, src + (size_t)from * row_bytes,
             row_bytes);
    }
  }
  return REF_OK;
}

static double row_value(int dtype, const void *rows, size_t at) {
  return dtype == REF_DT_F32 ? (double)((const float *)rows)[at]
                             : bf16_value(((const uint16_t *)rows)[at]);
}

static void store_value(int dtype, void *rows, size_t at, double v) {
  if (dtype == REF_DT_F32)
    ((float *)rows)[at] = (float)v;
  else
    ((uint16_t *)rows)[at] = moe_ref_f64_to_bf16(v);
}

/* Reverse of leg 2, on the node: for every (t, n) with a slot,
 *   part[node_slot[t*N+n], h] = sum over k with node(e(t,k)) = n of
 *                                w[t,k] * s[e(t,k)] * y[slot_pos[t,k], h]
 * summed in fp64 in k order (s = 1 when expert_scale is NULL).  part_exact
 * (may be NULL) gets the unrounded sums, part (may be NULL) the sums rounded
 * to nearest-even in part_dtype. */
int moe_ref_combine_partial(int T, int H, int E, int K, int R, int N,
                            int y_dtype, const void *y,
                            const int32_t *slot_pos, const float *topk_w,
                            const int32_t *topk_idx,
                            const float *expert_scale,
                            const int32_t *node_slot, int D, int part_dtype,
                            void *part, double *part_exact) {
  if (T < 0 || H < 1 || E < 1 || K < 1 || R < 1 || N < 1) return REF_EINVAL;
  if (E % R != 0 || R % N != 0) return REF_EINVAL;
  const int per_rank = E / R, per_node = R / N;
  for (int t = 0; t < T; ++t) {
    for (int n = 0; n < N; ++n) {
      int32_t p = node_slot[(size_t)t * N + n];
      if (p < 0) continue;
      if (p >= D) return REF_EINVAL;
      for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
          size_t i = (size_t)t * K + k;
          int e = topk_idx[i];
          if ((e / per_rank) / per_node != n) continue;
          double c = (double)topk_w[i];
          if (expert_scale) c *= (double)expert_scale[e];
          acc += c * row_value(y_dtype, y, (size_t)slot_pos[i] * H + h);
        }
        size_t o = (size_t)p * H + h;
        if (part_exact) part_exact[o] = acc;
        if (part) store_value(part_dtype, part, o, acc);
      }
    }
  }
  return REF_OK;
}

/* The same partials as the fp32 value a kernel stores before its one
 * rounding to part_dtype.  Reading of "the fp32 sum of the token's weighted
 * expert outputs on that node" ("MoX: Efficient MoE Routing on
 * Direct-Connect Topologies", Section 2.5: a node reduces the expert outputs
 * it holds before forwarding one vector): the coefficient is the fp32
 * product c = w[t,k] * s[e(t,k)], and the sum is the chain acc <- fma(c,
 * y, acc) from acc = +0 over the node's slots in ascending k, every step
 * rounded once to fp32.  It fixes which fp32 value a 16-bit partial is
 * rounded from, so both sides take that rounding decision in the same
 * precision.  Slots with slot_pos < 0 add nothing.  part_f32 (may be NULL)
 * gets the fp32 sums, part (may be NULL) those sums rounded to nearest-even
 * in part_dtype. */
int moe_ref_combine_partial_f32(int T, int H, int E, int K, int R, int N,
                                int y_dtype, const void *y,
                                const int32_t *slot_pos, const float *topk_w,
                                const int32_t *topk_idx,
                                const float *expert_scale,
                                const int32_t *node_slot, int D,
                                int part_dtype, void *part, float *part_f32) {
  if (T < 0 || H < 1 || E < 1 || K < 1 || R < 1 || N < 1) return REF_EINVAL;
  if (E % R != 0 || R % N != 0) return REF_EINVAL;
  const int per_rank = E / R, per_node = R / N;
  for (int t = 0; t < T; ++t) {
    for (int n = 0; n < N; ++n) {
      int32_t p = node_slot[(size_t)t * N + n];
      if (p < 0) continue;
      if (p >= D) return REF_EINVAL;
      for (int h = 0; h < H; ++h) {
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
          size_t i = (size_t)t * K + k;
          int e = topk_idx[i];
          if ((e / per_rank) / per_node != n || slot_pos[i] < 0) continue;
          float c = topk_w[i];
          if (expert_scale) c = c * expert_scale[e];
          float v = (float)row_value(y_dtype, y, (size_t)slot_pos[i] * H + h);
          acc = fmaf(c, v, acc);
        }
        size_t o = (size_t)p * H + h;
        if (part_f32) part_f32[o] = acc;
        if (part) store_value(part_dtype, part, o, (double)acc);
      }
    }
  }
  return REF_OK;
}

/* Reverse of leg 1, at the source: out[t, h] = sum over n with a slot of
 * part[node_slot[t*N+n], h], in fp64 in node order.  out_exact (may be NULL)
 * gets the unrounded sums, out (may be NULL) the sums rounded to
 * nearest-even in out_dtype. */
int moe_ref_combine_nodes(int T, int H, int N, int part_dtype,
                          const void *part, int D, const int32_t *node_slot,
                          int out_dtype, void *out, double *out_exact) {
  if (T < 0 || H < 1 || N < 1) return REF_EINVAL;
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int n = 0; n < N; ++n) {
        int32_t p = node_slot[(size_t)t * N + n];
        if (p < 0) continue;
        if (p >= D) return REF_EINVAL;
        acc += row_value(part_dtype, part, (size_t)p * H + h);
      }
      size_t o = (size_t)t * H + h;
      if (out_exact) out_exact[o] = acc;
      if (out) store_value(out_dtype, out, o, acc);
    }
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* 6. FP8 dispatch with per-block scales                                    */
/* ------------------------------------------------------------------------ */
/*
 * "Efficient and portable mixture-of-experts communication", sections
 * "Envío (Dispatch)" and "Combinación (Combine)": the dispatch sends tokens
 * with block scale factors (a quantised payload), the combine sends 16-bit
 * activations and forms the weighted average.  "Workload-Static Optical
 * Circuit Switching for Scalable LLM Inference Decode", section
 * "Communication precision": FP8 is supported for MoE dispatch.  The pages
 * name neither the 8-bit format nor the block size; the readings taken here:
 *   - codes are OCP FP8 E4M3: 1 sign bit, 4 exponent bits with bias 7, 3
 *     mantissa bits, subnormals below 2^-6, no infinities, largest finite
 *     magnitude 448 (exponent 15 with mantissa 7 is NaN); round to nearest,
 *     ties to even; the sign of the input is kept (also on zero);
 *   - every block of B consecutive elements of a row has one fp32 scale
 *     s = amax / 448 (amax = largest magnitude in the block), and its codes
 *     are e4m3(x * r) with r = 448 / amax; both quotients and the product
 *     are fp32 operations (round to nearest-even), so the integer codes are
 *     decided in the precision the kernel uses; a block of zeros has s = 0
 *     and zero codes;
 *   - a packed row is H code bytes followed by the H/B scales (fp32, little
 *     endian), zero-padded to a multiple of 128 bytes so that every row
 *     starts on a 128-byte boundary and no two rows share a 128-byte block:
 *     round_up(H + 4H/B, 128) bytes;
 *   - dequantised value = code value * s.
 */

/* Value of an E4M3 code (exact; NaN codes return NaN). */
double moe_ref_e4m3_value(uint8_t c) {
  int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
  if (ex == 15 && man == 7) return NAN;
  double mag = ex == 0 ? ldexp((double)man, -9)          /* man/8 * 2^-6 */
                       : ldexp(8.0 + man, ex - 7 - 3);   /* (1+man/8) 2^(ex-7) */
  return sign ? -mag : mag;
}

/* E4M3 code of v: magnitude clamped to 448, then rounded to the nearest
 * representable value with ties to the even mantissa. */
uint8_t moe_ref_e4m3_code(double v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  if (a > 448.0) a = 448.0;
  uint8_t code;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: multiples of 2^-9; 2^-6 itself is the first normal */
    double m = nearbyint(ldexp(a, 9)); /* 0..8, ties to even */
    code = (uint8_t)m;                 /* m == 8 encodes 2^-6 (exp 1, man 0) */
  } else {
    int e;
    (void)frexp(a, &e);                /* a = f 2^e, 0.5 <= f < 1 */
    e -= 1;                            /* a in [2^e, 2^(e+1)) */
    double m = nearbyint(ldexp(a, 3 - e)); /* 8..16, ties to even */
    if (m == 16.0) {
      m = 8.0;
      e += 1;
    }
    code = (uint8_t)(((e + 7) << 3) | ((int)m - 8));
  }
  return (uint8_t)(code | (neg << 7));
}

static float row_value_f32(int dtype, const void *rows, size_t at) {
  if (dtype == REF_DT_F32) return ((const float *)rows)[at];
  uint32_t u = (uint32_t)((const uint16_t *)rows)[at] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Quantise one row of H elements (x_dtype) into codes[H] and scales[H/B]. */
static void quant_row(int H, int B, int x_dtype, const void *x, size_t row,
                      uint8_t *codes, float *scales) {
  for (int b0 = 0; b0 < H; b0 += B) {
    float amax = 0.0f;
    for (int i = b0; i < b0 + B; ++i) {
      float v = fabsf(row_value_f32(x_dtype, x, row * H + i));
      if (v > amax) amax = v;
    }
    volatile float s = amax / 448.0f; /* fp32 quotient */
    scales[b0 / B] = s;
    if (amax == 0.0f) {
      for (int i = b0; i < b0 + B; ++i)
        codes[i] = signbit(row_value_f32(x_dtype, x, row * H + i)) ? 0x80 : 0;
      continue;
    }
    volatile float r = 448.0f / amax; /* fp32 quotient */
    for (int i = b0; i < b0 + B; ++i) {
      volatile float p = row_value_f32(x_dtype, x, row * H + i) * r;
      codes[i] = moe_ref_e4m3_code((double)p);
    }
  }
}

/* Row bytes of the FP8 send buffer: H codes + H/B fp32 scales, rounded up
 * to a multiple of 128. */
size_t moe_ref_fp8_row_bytes(int H, int B) {
  return ((size_t)H + 4 * (size_t)(H / B) + 127) & ~(size_t)127;
}

/* Pack with quantisation: every token's row is quantised once and written
 * to its K send rows: send[slot_pos[t*K+k]] = codes(x[t]) | scales(x[t]). */
int moe_ref_pack_fp8(int T, int K, int H, int B, int x_dtype, const void *x,
                     const int32_t *slot_pos, void *send) {
  if (T < 0 || K < 1 || H < 1 || B < 1 || H % B != 0) return REF_EINVAL;
  const size_t rb = moe_ref_fp8_row_bytes(H, B);
  unsigned char *dst = (unsigned char *)send;
  uint8_t codes[65536];
  float scales[65536];
  if (H > 65536) return REF_EINVAL;
  for (int t = 0; t < T; ++t) {
    quant_row(H, B, x_dtype, x, (size_t)t, codes, scales);
    for (int k = 0; k < K; ++k) {
      int32_t s = slot_pos[(size_t)t * K + k];
      if (s < 0 || (size_t)s >= (size_t)T * K) return REF_EINVAL;
      unsigned char *row = dst + (size_t)s * rb;
      memset(row, 0, rb);
      memcpy(row, codes, (size_t)H);
      memcpy(row + H, scales, sizeof(float) * (size_t)(H / B));
    }
  }
  return REF_OK;
}

/* Dequantised value of element h of an FP8 row. */
static double fp8_row_value(const unsigned char *row, int H, int B, int h) {
  float s;
  memcpy(&s, row + H + 4 * (size_t)(h / B), sizeof s);
  return moe_ref_e4m3_value(row[h]) * (double)s;
}

/* Combine of FP8 rows: out[t,h] = sum_k w[t,k] s[e(t,k)] deq(y[slot_pos[t,k]], h)
 * in fp64, k order; out_exact (may be NULL) unrounded, out (may be NULL)
 * rounded to nearest-even in out_dtype. */
int moe_ref_combine_fp8(int T, int H, int K, int B, const void *y,
                        const int32_t *slot_pos, const float *topk_w,
                        const int32_t *topk_idx, const float *expert_scale,
                        int out_dtype, void *out, double *out_exact) {
  if (T < 0 || H < 1 || K < 1 || B < 1 || H % B != 0) return REF_EINVAL;
  if (expert_scale && !topk_idx) return REF_EINVAL;
  const size_t rb = moe_ref_fp8_row_bytes(H, B);
  const unsigned char *src = (const unsigned char *)y;
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k) {
        size_t i = (size_t)t * K + k;
        double c = (double)topk_w[i];
        if (expert_scale) c *= (double)expert_scale[topk_idx[i]];
        acc += c * fp8_row_value(src + (size_t)slot_pos[i] * rb, H, B, h);
      }
      size_t o = (size_t)t * H + h;
      if (out_exact) out_exact[o] = acc;
      if (out) store_value(out_dtype, out, o, acc);
    }
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* 7. Capacity-padded and bucketed layout                                   */
/* ------------------------------------------------------------------------ */
/*
 * "Workload-Static Optical Circuit Switching for Scalable LLM Inference
 * Decode", section "Variable MoE Traffic and Regularization": each expert
 * gets a fixed capacity (capacity factor gamma >= 1) and every buffer between
 * a source group and a destination expert is padded to that many rows, so
 * every step exchanges the same volume; tokens beyond the capacity leave on an
 * overflow path (dropped here).  Bucketing generalises this: per-pair counts
 * are rounded up to one of q levels C_1 < ... < C_q.  The capacity formula
 * itself is missing from the page; the reading taken is
 * C = ceil(gamma * T * K / E).
 *
 * With levels[0..q-1] ascending and Cmax = levels[q-1]:
 *   kept_e = min(count_e, Cmax), the first kept_e tokens of expert e in
 *            token order (the same (t, k) walk as the dropless layout);
 *   cap_e  = the smallest level >= kept_e (q = 1: every expert gets C rows);
 *   expert_off[E+1] = exclusive prefix of cap_e; expert e's rows are
 *            [expert_off[e], expert_off[e] + cap_e), the first kept_e used;
 *   slot_pos[t*K+k] = expert_off[e] + rank of t among e's tokens, or -1 when
 *            the rank is >= Cmax (dropped);
 *   row_src[r] = t*K+k for used rows, -1 for padding rows (E*Cmax entries);
 *   dropped = sum_e (count_e - kept_e).
 */
int moe_ref_layout_capacity(int T, int E, int K, const int32_t *topk_idx,
                            const int32_t *levels, int q,
                            int32_t *expert_count, int32_t *expert_cap,
                            int32_t *expert_off, int32_t *slot_pos,
                            int32_t *row_src, int32_t *dropped) {
  if (T < 0 || E < 1 || K < 1 || q < 1) return REF_EINVAL;
  for (int j = 0; j < q; ++j)
    if (levels[j] < 1 || (j > 0 && levels[j] <= levels[j - 1]))
      return REF_EINVAL;
  const int32_t cmax = levels[q - 1];
  const size_t TK = (size_t)T * K;
  for (size_t i = 0; i < TK; ++i)
    if (topk_idx[i] < 0 || topk_idx[i] >= E) return REF_EINVAL;
  for (int e = 0; e < E; ++e) expert_count[e] = 0;
  for (size_t i = 0; i < TK; ++i) expert_count[topk_idx[i]] += 1;
  int32_t drop = 0;
  expert_off[0] = 0;
  for (int e = 0; e < E; ++e) {
    int32_t kept = expert_count[e] < cmax ? expert_count[e] : cmax;
    drop += expert_count[e] - kept;
    int32_t cap = cmax;
    for (int j = q - 1; j >= 0; --j)
      if (levels[j] >= kept) cap = levels[j];
    expert_cap[e] = cap;
    expert_off[e + 1] = expert_off[e] + cap;
  }
  *dropped = drop;
  for (size_t r = 0; r < (size_t)E * cmax; ++r) row_src[r] = -1;
  int32_t cursor[8192];
  if (E > 8192) return REF_EINVAL;
  for (int e = 0; e < E; ++e) cursor[e] = 0;
  for (size_t i = 0; i < TK; ++i) {
    int e = topk_idx[i];
    int32_t rank = cursor[e]++;
    if (rank < cmax) {
      slot_pos[i] = expert_off[e] + rank;
      row_src[slot_pos[i]] = (int32_t)i;
    } else {
      slot_pos[i] = -1;
    }
  }
  return REF_OK;
}

/* Pack into a capacity-padded buffer of n_rows rows: a used row is the x row
 * of its token (row_src / K), a padding row (row_src < 0) is zero. */
int moe_ref_pack_capacity(int T, int K, size_t row_bytes, const void *x,
                          const int32_t *row_src, int n_rows, void *send) {
  if (T < 0 || K < 1 || n_rows < 0) return REF_EINVAL;
  const unsigned char *src = (const unsigned char *)x;
  unsigned char *dst = (unsigned char *)send;
  for (int r = 0; r < n_rows; ++r) {
    int32_t i = row_src[r];
    if (i < 0) {
      memset(dst + (size_t)r * row_bytes, 0, row_bytes);
    } else {
      if ((size_t)i >= (size_t)T * K) return REF_EINVAL;
      memcpy(dst + (size_t)r * row_bytes, src + (size_t)(i / K) * row_bytes,
             row_bytes);
    }
  }
  return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* 8. Communication-aware task assignment                                   */
/* ------------------------------------------------------------------------ */
/*
 * "Cobalt: Leveraging Expert Co-activation for Efficient Distributed MoE
 * Training", Section 3.3 (Algorithm 1).  G ranks on N nodes, G/N contiguous
 * ranks per node; holds[r*E + e] != 0 when rank r has a replica of expert e.
 * For token t with source rank src_rank[t] on node sn:
 *   Step 1: a selected expert with a replica on node sn runs on node sn; the
 *   others (the set U) need remote nodes.  For e in U, m_e = the remote
 *   nodes holding e.  A mask b of remote nodes is feasible when b & m_e != 0
 *   for every e in U; the chosen b is a feasible mask of smallest popcount
 *   (the minimum set cover), and among those the one of smallest value (the
 *   page does not say which; masks are enumerated by popcount, then value).
 *   Each e in U runs on a node drawn from b & m_e.
 *   Step 2: the rank is drawn from the ranks of that node holding e.
 * Random draws are inputs: a draw u (uint32) picks entry floor(u * c / 2^32)
 * of a list of c candidates in ascending order.
 * Outputs: assign_rank[t*K+k], remote_mask[t] = b.  Returns REF_EINVAL when
 * an expert has no replica at all or a shape is bad.
 */
static int pick(uint32_t u, int c) {
  return (int)(((uint64_t)u * (uint64_t)c) >> 32);
}

int moe_ref_assign(int T, int E, int K, int G, int N, const int32_t *topk_idx,
                   const int32_t *src_rank, const uint8_t *holds,
                   const uint32_t *u_node, const uint32_t *u_rank,
                   int32_t *assign_rank, uint64_t *remote_mask) {
  /* the oracle scans all 2^N masks: small N only */
  if (T < 0 || E < 1 || K < 1 || G < 1 || N < 1 || N > 24 || G % N != 0)
    return REF_EINVAL;
  const int per_node = G / N;
  for (int t = 0; t < T; ++t) {
    const int sr = src_rank[t];
    if (sr < 0 || sr >= G) return REF_EINVAL;
    const int sn = sr / per_node;
    uint64_t m[64];   /* remote nodes holding each selected expert */
    int in_u[64];
    if (K > 64) return REF_EINVAL;
    int n_u = 0;
    for (int k = 0; k < K; ++k) {
      const int e = topk_idx[(size_t)t * K + k];
      if (e < 0 || e >= E) return REF_EINVAL;
      uint64_t nodes = 0;
      for (int r = 0; r < G; ++r)
        if (holds[(size_t)r * E + e]) nodes |= (uint64_t)1 << (r / per_node);
      if (nodes == 0) return REF_EINVAL;
      in_u[k] = !((nodes >> sn) & 1);
      m[k] = nodes & ~((uint64_t)1 << sn);
      n_u += in_u[k];
    }
    /* Step 1: smallest-popcount feasible mask, then smallest value: scan
     * every mask of popcount p (bit sn clear) in increasing value */
    uint64_t best = 0;
    if (n_u > 0) {
      int found = 0;
      for (int p = 1; p <= N - 1 && !found; ++p) {
        for (uint64_t b = 1; b < ((uint64_t)1 << N); ++b) {
          if (__builtin_popcountll(b) != p || ((b >> sn) & 1)) continue;
          int ok = 1;
          for (int k = 0; k < K && ok; ++k)
            if (in_u[k] && !(b & m[k])) ok = 0;
          if (ok) {
            best = b;
            found = 1;
            break;
          }
        }
      }
      if (!found) return REF_EINVAL;
    }
    remote_mask[t] = best;
    for (int k = 0; k < K; ++k) {
      const size_t i = (size_t)t * K + k;
      const int e = topk_idx[i];
      int node = sn;
      if (in_u[k]) {
        uint64_t cand = best & m[k];
        int j = pick(u_node[i], __builtin_popcountll(cand));
        for (int n = 0; n < N; ++n)
          if ((cand >> n) & 1) {
            if (j == 0) {
              node = n;
              break;
            }
            --j;
          }
      }
      /* Step 2: uniform among node's ranks holding e, ascending */
      int c = 0;
      for (int r = node * per_node; r < (node + 1) * per_node; ++r)
        c += holds[(size_t)r * E + e] != 0;
      int j = pick(u_rank[i], c);
      int rank = -1;
      for (int r = node * per_node; r < (node + 1) * per_node; ++r)
        if (holds[(size_t)r * E + e]) {
          if (j == 0) {
            rank = r;
            break;
          }
          --j;
        }
      assign_rank[i] = rank;
    }
  }
  return REF_OK;
}
