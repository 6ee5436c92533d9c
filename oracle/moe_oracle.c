/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU reference of the single-GPU
 * Mixture-of-Experts path: route -> dispatch (layout + row scatter) -> SwiGLU
 * expert FFN -> probability-weighted combine, and the combine's backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  The GPU library
 * shares no code, header, table or helper with it.
 *
 * Arithmetic: fp64 unless a step fixes another precision:
 *   - router weights: softmax and renormalisation in double, one rounding to fp32;
 *   - combine: fp32 fused multiply-add accumulation in top-k slot order (the
 *     required "fp32 combine accumulation"), one rounding to the output type;
 *   - expert FFN: double accumulation, bf16 rounding of the SwiGLU intermediate
 *     and of the output (both are bf16 tensors in the method);
 *   - combine backward: double, one rounding per stored value;
 *   - expert FFN backward (oracle/__init__.py, numpy fp64 matmuls per expert):
 *     double throughout, one rounding per stored value.
 * Compiled with -O2 -ffp-contract=off so no fused operation appears that the
 * source does not write.
 *
 * Sources (the web pages this path is built from):
 *   [MEG]  "Megatron MoE 实现" (Megatron MoE implementation), MoELayer.forward and
 *          its four stages: router -> (probs, routing_map), dispatch_preprocess,
 *          dispatch_postprocess -> (dispatched_input, tokens_per_expert,
 *          permuted_probs), experts, combine_postprocess.
 *   [MORI] ROCm/Megatron-LM pull request "Add MORI as a Token Dispatcher", commit
 *          log: -1 sentinels for non-local experts, multihot routing map,
 *          sync-free per-expert counts, fixed-size buffers with masked tails.
 *   [DS]   DeepSpeed deepspeed/moe/ep_tp_dispatch.py: RoutedAssignmentPayload
 *          (capacity_slots, drop_mask, pad_mask), assignment_ordinals_by_expert
 *          (stable ordinals within expert segments), restore_combined (weighted
 *          rows added one top-k slot at a time into a zeroed output).
 *   [HT]   mscclpp commit "high-throughput MoE dispatch/combine", Validation
 *          (e256 / top-8 / hidden 7168 / 4096 tokens, exact dispatch/combine).
 * The router arithmetic (softmax, top-k with lowest-index tie-break,
 * renormalisation), the capacity factor and the SwiGLU expert are fixed by the
 * workload definitions, not by the pages; each reading is stated where used.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DT_F32 0
#define DT_BF16 1

/* ------------------------------------------------------------------ formats */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> double: a bf16 is the top half of an fp32, so the widening is exact. */
static double bf16_value(uint16_t h) { return (double)f32_from_bits((uint32_t)h << 16); }

/* double -> bf16, round to nearest, ties to even, in one rounding.  bf16 keeps
 * 8 significant bits; below 2^-126 the spacing is fixed at 2^-133. */
static uint16_t bf16_round(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e);                       /* 2^(e-1) <= a < 2^e */
  int q = e - 8;                      /* exponent of the last kept bit */
  if (q < -133) q = -133;
  double r = ldexp(nearbyint(ldexp(a, -q)), q);   /* nearbyint: ties to even */
  if (r >= 0x1p128) return sign | 0x7F80;
  return sign | (uint16_t)(bits_from_f32((float)r) >> 16);   /* (float)r is exact */
}

/* Read element i of an activation tensor of type dt as a double (exact). */
static double act_load(const void *p, int dt, int64_t i) {
  if (dt == DT_F32) return (double)((const float *)p)[i];
  return bf16_value(((const uint16_t *)p)[i]);
}

/* Store a double into an activation tensor of type dt with one rounding. */
static void act_store(void *p, int dt, int64_t i, double v) {
  if (dt == DT_F32) ((float *)p)[i] = (float)v;
  else ((uint16_t *)p)[i] = bf16_round(v);
}

/* ------------------------------------------------------------------- route */

/* Selection order on experts of one token: expert a comes before expert b when
 * its logit is larger, or the logits are equal and a < b (lowest-index
 * tie-break).  -0.0 and +0.0 compare equal (C's == does that); a NaN logit
 * comes after every number. */
static int selected_before(float va, int a, float vb, int b) {
  int na = isnan(va), nb = isnan(vb);
  if (na || nb) {
    if (na && nb) return a < b;
    return nb;
  }
  if (va > vb) return 1;
  if (va < vb) return 0;
  return a < b;
}

/* Router [MEG MoELayer.forward, stage 1: probs, routing_map = router(hidden)].
 * Per token: the k experts first in selection order, stored largest first;
 * probabilities p = softmax over all E logits (double); the k chosen are
 * renormalised, w_j = p_j / sum_j' p_j', and rounded once to fp32; the routing
 * map is the multihot [N, E] row ([MORI] multihot conversion); tokens_per_expert
 * is the column sum of the map.  token_mask (nullable): nonzero marks a
 * padding token, routed nowhere.  expert_bias (nullable, [E]): a
 * selection-only bias -- experts are ranked by logit + bias (fp32), the
 * weights still come from the logits alone (the load-balancing expert bias
 * of Megatron's router that the UltraEP pull request lists as not yet
 * supported there). */
int oracle_route(int64_t n, int e, int k, const float *logits, const float *expert_bias, const uint8_t *token_mask,
                 int32_t *topk_idx, float *topk_w, uint8_t *routing_map, int32_t *tokens_per_expert) {
  if (n < 0 || e < 1 || k < 1 || k > e) return -1;
  char *taken = (char *)malloc((size_t)e);
  double *p = (double *)malloc(sizeof(double) * (size_t)e);
  float *sc = (float *)malloc(sizeof(float) * (size_t)e);
  if (!taken || !p || !sc) { free(taken); free(p); free(sc); return -2; }
  if (tokens_per_expert) memset(tokens_per_expert, 0, sizeof(int32_t) * (size_t)e);
  for (int64_t t = 0; t < n; ++t) {
    const float *l = logits + t * e;
    memset(taken, 0, (size_t)e);
    if (token_mask && token_mask[t]) {
      /* a padding token takes part in no routing [MORI router: padding tokens
       * masked out of routing and dispatch]: every slot is the -1 sentinel with
       * weight 0, its map row is empty and it is not counted */
      for (int j = 0; j < k; ++j) { topk_idx[t * k + j] = -1; topk_w[t * k + j] = 0.0f; }
      if (routing_map) memset(routing_map + t * e, 0, (size_t)e);
      continue;
    }
    /* selection score: the logit, plus the expert's bias when one is given
     * (an fp32 sum); the weights below use the logits alone */
    for (int x = 0; x < e; ++x) sc[x] = expert_bias ? l[x] + expert_bias[x] : l[x];
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int x = 0; x < e; ++x) {
        if (taken[x]) continue;
        if (best < 0 || selected_before(sc[x], x, sc[best], best)) best = x;
      }
      taken[best] = 1;
      topk_idx[t * k + j] = best;
    }
    double m = -INFINITY;
    for (int x = 0; x < e; ++x) if ((double)l[x] > m) m = (double)l[x];
    double z = 0.0;
    for (int x = 0; x < e; ++x) { p[x] = exp((double)l[x] - m); z += p[x]; }
    for (int x = 0; x < e; ++x) p[x] /= z;
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += p[topk_idx[t * k + j]];
    for (int j = 0; j < k; ++j) topk_w[t * k + j] = (float)(p[topk_idx[t * k + j]] / s);
    if (routing_map) for (int x = 0; x < e; ++x) routing_map[t * e + x] = (uint8_t)taken[x];
    if (tokens_per_expert) for (int x = 0; x < e; ++x) tokens_per_expert[x] += taken[x];
  }
  free(taken);
  free(p);
  free(sc);
  return 0;
}

/* ---------------------------------------------- random (balanced) logits */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): ten rounds of two
 * 32x32 -> 64-bit multiplications (multipliers 0xD2511F53 and 0xCD9E8D57),
 * the key bumped by the Weyl constants 0x9E3779B9 and 0xBB67AE85 between
 * rounds.  out = Philox(counter ctr[4], key key[2]). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Random router logits for the force-balanced benchmark mode (the UltraEP pull
 * request "Integrate UltraEP Runtime": random-logits routing for balanced
 * benchmark runs).  logit[t, x] = (w >> 8) * 2^-24, a uniform number in [0, 1)
 * exact in fp32, where w is word x % 4 of Philox4x32-10 with counter
 * (x / 4, t mod 2^32, t / 2^32, 0) and key (seed mod 2^32, seed / 2^32). */
void oracle_random_logits(int64_t n, int e, uint64_t seed, float *logits) {
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  for (int64_t t = 0; t < n; ++t)
    for (int x = 0; x < e; ++x) {
      const uint32_t ctr[4] = {(uint32_t)(x / 4), (uint32_t)t, (uint32_t)((uint64_t)t >> 32), 0u};
      uint32_t w[4];
      oracle_philox4x32_10(ctr, key, w);
      logits[t * e + x] = (float)(w[x % 4] >> 8) * (1.0f / 16777216.0f);
    }
}

/* ------------------------------------------------------------------ layout */

/* Rows of the permuted buffer: E*C with a capacity, else max_rows if given,
 * else one row per assignment. */
int64_t oracle_layout_rows(int64_t n, int k, int e, int capacity, int64_t max_rows, int row_align) {
  if (capacity > 0) return (int64_t)e * capacity;
  if (max_rows > 0) return max_rows;
  /* every segment rounded up to row_align rows adds at most row_align - 1 pad rows */
  return n * k + (row_align > 1 ? (int64_t)e * (row_align - 1) : 0);
}

/* Dispatch layout [MEG dispatch_preprocess / dispatch_postprocess; DS
 * RoutedAssignmentPayload and assignment_ordinals_by_expert; MORI sentinels].
 * Assignment a = t*k + j goes to expert topk_idx[a]; -1 is a non-local slot and is
 * skipped; ids < -1 or >= E are invalid, skipped and counted.
 *  - ordinal[a]: number of earlier assignments (smaller a) to the same expert
 *    (a stable counting sort by expert; equals the segment-start/cummax ordinal
 *    of the stably expert-sorted list).
 *  - capacity C > 0: segment of expert e starts at e*C, the first C assignments
 *    (by ordinal) are kept, the rest dropped; slots kept_e..C-1 are pad rows.
 *    C <= 0: segments are the exclusive scan of the counts, each rounded up to
 *    a multiple of row_align rows when row_align > 1 ([MORI] padding routing
 *    maps / FP8 padding: every expert's segment starts on an aligned row),
 *    clipped to the row budget; assignments past the budget are dropped; the
 *    rows between an expert's kept rows and the next segment are pad rows.
 *  - drop_policy (capacity only): 0 keeps the first C assignments of an
 *    expert by position, as above; 1 keeps the C with the largest weights
 *    topk_w[a] (ties: the earlier assignment; NaN below every number),
 *    Megatron's "probs" token-drop policy.
 *  - assign_row[a] = offset[e] + (the number of kept assignments of e before a)
 *    when kept, else -1 (= offset[e] + ordinal[a] under the position policy).
 *  - row_src[r] = the assignment placed in row r, else -1; pad_mask[r] = 1 for
 *    every row that holds no assignment (capacity pad or unused tail).
 *  - counters = {kept, dropped, pad rows (capacity or alignment), invalid ids}. */
/* Drop-policy order of two assignments of one expert: the larger weight first,
 * NaN after every number, -0.0 == +0.0; equal weights keep position order. */
static const float *g_sort_w;
static int by_weight_desc(const void *pa, const void *pb) {
  const int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
  const float va = g_sort_w[a], vb = g_sort_w[b];
  const int na = isnan(va), nb = isnan(vb);
  if (na != nb) return na ? 1 : -1;
  if (!na) {
    if (va > vb) return -1;
    if (va < vb) return 1;
  }
  return a < b ? -1 : (a > b ? 1 : 0);
}

int oracle_layout(int64_t n, int k, int e, int capacity, int64_t max_rows, int row_align, int drop_policy,
                  const int32_t *topk_idx, const float *topk_w, int32_t *tokens_per_expert, int32_t *expert_offsets, int32_t *ordinal,
                  int32_t *assign_row, int32_t *row_src, uint8_t *drop_mask, uint8_t *pad_mask,
                  int32_t *counters) {
  if (n < 0 || k < 1 || e < 1) return -1;
  int64_t a_total = n * k;
  int64_t rows = oracle_layout_rows(n, k, e, capacity, max_rows, row_align);
  const int64_t align = row_align > 1 ? row_align : 1;
  int64_t *count = (int64_t *)calloc((size_t)e, sizeof(int64_t));
  int64_t *seen = (int64_t *)calloc((size_t)e, sizeof(int64_t));
  int64_t *kept = (int64_t *)calloc((size_t)e, sizeof(int64_t));
  if (!count || !seen || !kept) { free(count); free(seen); free(kept); return -2; }
  int64_t invalid = 0;
  for (int64_t a = 0; a < a_total; ++a) {
    int32_t x = topk_idx[a];
    if (x == -1) continue;
    if (x < -1 || x >= e) { ++invalid; continue; }
    ++count[x];
  }
  if (capacity > 0) {
    for (int x = 0; x < e; ++x) {
      expert_offsets[x] = (int32_t)((int64_t)x * capacity);
      kept[x] = count[x] < capacity ? count[x] : capacity;
    }
    expert_offsets[e] = (int32_t)rows;
  } else {
    int64_t off = 0;
    for (int x = 0; x < e; ++x) {
      expert_offsets[x] = (int32_t)(off < rows ? off : rows);
      off += (count[x] + align - 1) / align * align;
    }
    expert_offsets[e] = (int32_t)(off < rows ? off : rows);
    for (int x = 0; x < e; ++x) {
      const int64_t room = rows - expert_offsets[x];
      kept[x] = count[x] < room ? count[x] : room;
    }
  }
  /* keep[a]: under the probs policy, sort each over-full expert's assignments
   * by weight and keep the first C; otherwise keep by position (ordinal < kept) */
  uint8_t *keep = NULL;
  if (capacity > 0 && drop_policy == 1) {
    keep = (uint8_t *)calloc((size_t)(a_total > 0 ? a_total : 1), 1);
    int64_t *list = (int64_t *)malloc(sizeof(int64_t) * (size_t)(a_total > 0 ? a_total : 1));
    if (!keep || !list) { free(keep); free(list); free(count); free(seen); free(kept); return -2; }
    g_sort_w = topk_w;
    for (int x = 0; x < e; ++x) {
      int64_t m = 0;
      for (int64_t a = 0; a < a_total; ++a)
        if (topk_idx[a] == x) list[m++] = a;
      if (m > capacity) qsort(list, (size_t)m, sizeof(int64_t), by_weight_desc);
      for (int64_t i = 0; i < m && i < capacity; ++i) keep[list[i]] = 1;
    }
    free(list);
  }
  int64_t *placed = (int64_t *)calloc((size_t)e, sizeof(int64_t));
  if (!placed) { free(keep); free(count); free(seen); free(kept); return -2; }
  for (int64_t r = 0; r < rows; ++r) { row_src[r] = -1; pad_mask[r] = 1; }
  int64_t dropped = 0, kept_total = 0;
  for (int64_t a = 0; a < a_total; ++a) {
    int32_t x = topk_idx[a];
    drop_mask[a] = 0;
    if (x < 0 || x >= e) { ordinal[a] = -1; assign_row[a] = -1; continue; }
    int64_t o = seen[x]++;
    ordinal[a] = (int32_t)o;
    if (keep ? keep[a] : o < kept[x]) {
      int64_t r = expert_offsets[x] + placed[x]++;
      assign_row[a] = (int32_t)r;
      row_src[r] = (int32_t)a;
      pad_mask[r] = 0;
      ++kept_total;
    } else {
      assign_row[a] = -1;
      drop_mask[a] = 1;
      ++dropped;
    }
  }
  free(keep);
  free(placed);
  for (int x = 0; x < e; ++x) tokens_per_expert[x] = (int32_t)kept[x];
  counters[0] = (int32_t)kept_total;
  counters[1] = (int32_t)dropped;
  counters[2] = (int32_t)(expert_offsets[e] - kept_total);  /* rows below the used end holding nothing */
  counters[3] = (int32_t)invalid;
  free(count);
  free(seen);
  free(kept);
  return 0;
}

/* ----------------------------------------------------------------- scatter */

/* Row scatter [MEG dispatch_preprocess permutes hidden states and probs; HT
 * Validation: the dispatched copy is exact].  Each kept assignment's token row
 * is copied bit for bit into its row; its weight goes to w_perm.  Pad rows --
 * rows below pad_limit (expert_offsets[E]: the end of the last segment) that
 * hold no assignment, i.e. capacity or alignment pads -- are all-zero bits
 * with weight 0 ([MORI] masked tails are filled with 0).  Rows of an unused
 * dropless tail get weight 0 and keep their data. */
void oracle_scatter(int64_t n, int k, int64_t row_bytes, const uint8_t *x, const int32_t *assign_row,
                    const float *topk_w, int64_t rows, const int32_t *row_src, int64_t pad_limit,
                    uint8_t *x_perm, float *w_perm) {
  for (int64_t a = 0; a < n * k; ++a) {
    int32_t r = assign_row[a];
    if (r < 0) continue;
    memcpy(x_perm + (int64_t)r * row_bytes, x + (a / k) * row_bytes, (size_t)row_bytes);
    if (w_perm) w_perm[r] = topk_w[a];
  }
  for (int64_t r = 0; r < rows; ++r) {
    if (row_src[r] >= 0) continue;
    if (r < pad_limit) memset(x_perm + r * row_bytes, 0, (size_t)row_bytes);
    if (w_perm) w_perm[r] = 0.0f;
  }
}

static double silu(double z);

/* -------------------------------------------------------- MXFP8 dispatch */

/* FP8 dispatch ([MORI] commit log: optional FP8 dispatch, a per-token scale
 * tensor beside the quantised rows; the ROCm Megatron training script's MXFP8
 * recipe).  Read as MXFP8 as the OCP "Microscaling (MX) Formats Specification"
 * v1.0 defines it: each run of 32 consecutive elements of a row shares one
 * E8M0 scale X = 2^s (code s + 127, s in [-127, 127]); element i is stored as
 * the FP8 E4M3 code P_i of V_i / X.  The scale follows the specification's
 * conversion: s = floor(log2(max_i |V_i|)) - 8 (8 = the largest E4M3 exponent),
 * clipped to [-127, 127]; V_i / X is rounded to the nearest E4M3 value, ties
 * to even, and magnitudes above the largest finite E4M3 value (448) are
 * clamped to it.  An all-zero block is not covered by the formula (log2 0);
 * read: code 0, the smallest scale (every element is 0 under any scale).
 * Inputs must be finite. */

/* Value of the non-negative E4M3 code c (0 .. 0x7E; 0x7F is NaN): exponent
 * field e = c >> 3 (bias 7), mantissa m = c & 7; e = 0 is subnormal,
 * m/8 * 2^-6, else (1 + m/8) * 2^(e-7). */
static double e4m3_value(int c) {
  const int e = c >> 3, m = c & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

/* E4M3 code of v: |v| clamped to 448, then the nearest code by value (the
 * codes 0 .. 0x7E ascend in value), ties to the even code; sign bit = sign of v. */
static uint8_t e4m3_encode(double v) {
  double a = fabs(v);
  if (a > 448.0) a = 448.0;
  int c = 0, hi = 0x7E; /* bisection for the largest code not above a */
  while (c < hi) {
    const int mid = (c + hi + 1) / 2;
    if (e4m3_value(mid) <= a) c = mid;
    else hi = mid - 1;
  }
  if (c < 0x7E) {
    const double below = a - e4m3_value(c), above = e4m3_value(c + 1) - a;
    if (above < below || (above == below && (c & 1))) ++c;
  }
  return (uint8_t)(c | (signbit(v) ? 0x80 : 0));
}

/* MXFP8 of one bf16 row of h elements (h a multiple of 32). */
static void mx_quantize_row(int64_t h, const uint16_t *x, uint8_t *q, uint8_t *scale) {
  for (int64_t b = 0; b < h / 32; ++b) {
      const uint16_t *v = x + 32 * b;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs(bf16_value(v[i])) > amax) amax = fabs(bf16_value(v[i]));
      int s = -127;
      if (amax > 0.0) {
        int ex;
        frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
        s = ex - 1 - 8;
        if (s < -127) s = -127;
        if (s > 127) s = 127;
      }
      scale[b] = (uint8_t)(s + 127);
      for (int i = 0; i < 32; ++i) q[32 * b + i] = e4m3_encode(ldexp(bf16_value(v[i]), -s));
  }
}

/* MXFP8 quantisation of `rows` bf16 rows of h elements (h a multiple of 32):
 * q [rows, h] E4M3 codes, scale [rows, h/32] E8M0 codes. */
void oracle_mx_quantize(int64_t rows, int64_t h, const uint16_t *x, uint8_t *q, uint8_t *scale) {
  for (int64_t r = 0; r < rows; ++r) mx_quantize_row(h, x + r * h, q + r * h, scale + r * (h / 32));
}

/* Value of element i of an MXFP8 row: E4M3 code times 2^(scale code - 127). */
static double mx_value(const uint8_t *q, const uint8_t *scale, int64_t i) {
  const int c = q[i] & 0x7F;
  const double v = ldexp(e4m3_value(c), (int)scale[i / 32] - 127);
  return (q[i] & 0x80) ? -v : v;
}

/* The SwiGLU expert over MXFP8 operands (the expert FFN with FP8 grouped
 * experts: the dispatched rows as moe_dispatch_mxfp8 writes them, the weights
 * MXFP8 along their K dimension).  For a row r of expert e's segment, with
 * every operand value the exact value of its code and scale:
 *   g_i, u_i = sum_h x[r,h] W_gu[e, i, h], sum_h x[r,h] W_gu[e, I+i, h]  (double)
 *   a_i      = bf16(silu(g_i) * u_i)            (the bf16 intermediate)
 *   a'       = MXFP8 of the row a (blocks of 32 along I), dequantised
 *   y[r, c]  = bf16(sum_i a'_i W_d[e, c, i])                          (double)
 * The same listed-rows interface as oracle_expert_ffn_rows; xq [.., h], xs
 * [.., h/32]; wguq [E, 2I, h], wgus [E, 2I, h/32]; wdq [E, h, I], wds [E, h, I/32]. */
void oracle_expert_ffn_mxfp8_rows(int64_t nrows, const int64_t *rows, int e, int64_t h, int64_t inter,
                                  const uint8_t *xq, const uint8_t *xs, const int32_t *offsets,
                                  const int32_t *counts, const uint8_t *wguq, const uint8_t *wgus,
                                  const uint8_t *wdq, const uint8_t *wds, uint16_t *y_rows, int32_t *expert_of) {
  double *x = malloc(sizeof(double) * (size_t)h);
  uint16_t *a = malloc(sizeof(uint16_t) * (size_t)inter);
  uint8_t *aq = malloc((size_t)inter), *as = malloc((size_t)(inter / 32));
  for (int64_t j = 0; j < nrows; ++j) {
    const int64_t r = rows[j];
    int ex = -1;
    for (int x_ = 0; x_ < e; ++x_)
      if (r >= offsets[x_] && r < (int64_t)offsets[x_] + counts[x_]) ex = x_;
    expert_of[j] = ex;
    if (ex < 0) {
      memset(y_rows + j * h, 0, sizeof(uint16_t) * (size_t)h);
      continue;
    }
    for (int64_t c = 0; c < h; ++c) x[c] = mx_value(xq + r * h, xs + r * (h / 32), c);
    const int64_t gu_row = 2 * inter;
    for (int64_t i = 0; i < inter; ++i) {
      double g = 0.0, u = 0.0;
      const int64_t gi = (int64_t)ex * gu_row + i, ui = (int64_t)ex * gu_row + inter + i;
      for (int64_t c = 0; c < h; ++c) {
        g += x[c] * mx_value(wguq + gi * h, wgus + gi * (h / 32), c);
        u += x[c] * mx_value(wguq + ui * h, wgus + ui * (h / 32), c);
      }
      a[i] = bf16_round(silu(g) * u);
    }
    mx_quantize_row(inter, a, aq, as);
    for (int64_t c = 0; c < h; ++c) {
      const int64_t di = (int64_t)ex * h + c;
      double acc = 0.0;
      for (int64_t i = 0; i < inter; ++i)
        acc += mx_value(aq, as, i) * mx_value(wdq + di * inter, wds + di * (inter / 32), i);
      y_rows[j * h + c] = bf16_round(acc);
    }
  }
  free(x);
  free(a);
  free(aq);
  free(as);
}

/* Element-wise E4M3 encoding of n doubles (the element step alone, scale 1). */
void oracle_e4m3_encode_array(int64_t n, const double *v, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(v[i]);
}

/* Values of n E4M3 codes (0x7F / 0xFF give NaN). */
void oracle_e4m3_decode_array(int64_t n, const uint8_t *c, double *out) {
  for (int64_t i = 0; i < n; ++i) {
    const int m = c[i] & 0x7F;
    const double v = m == 0x7F ? NAN : e4m3_value(m);
    out[i] = (c[i] & 0x80) ? -v : v;
  }
}

/* ------------------------------------------------ hot-expert replication */

/* [UEP] InternLM/xtuner pull request "Integrate UltraEP Runtime": replicas of
 * hot experts created from the current load, part of their tokens rerouted to
 * the replica slots (logical -> physical placement and reroute), replica
 * weights synchronised from the masters, one grouped GEMM over master and
 * replica experts (weights from two storage bases), replica weight gradients
 * written to a replica buffer and reduced into the masters'.  The pages give
 * no placement or split rule; readings:
 *   placement: R slots filled one at a time, each going to the logical expert
 *     with the largest load per copy, count_e / (1 + slots_e) (ties: lowest e);
 *   reroute: expert e's count_e assignments, in assignment order, are cut into
 *     m_e = 1 + slots_e consecutive runs as equal as the count allows (run j
 *     holds ordinals ceil(j count/m) .. ceil((j+1) count/m) - 1); run 0 stays
 *     on the master, run j >= 1 goes to e's j-th slot in slot order.
 * Physical expert p < E is the master of logical expert p, p = E + i is slot i. */

/* Placement: replica_of[i] = logical expert of slot i, i = 0 .. r-1. */
void oracle_replica_plan(int e, const int32_t *counts, int r, int32_t *replica_of) {
  int *slots = calloc((size_t)e, sizeof(int));
  for (int i = 0; i < r; ++i) {
    int best = 0;
    for (int x = 1; x < e; ++x) /* counts[x]/(1+slots[x]) > counts[best]/(1+slots[best]), exactly */
      if ((int64_t)counts[x] * (1 + slots[best]) > (int64_t)counts[best] * (1 + slots[x])) best = x;
    replica_of[i] = best;
    ++slots[best];
  }
  free(slots);
}

/* Reroute of logical ids idx [n*k] to physical ids phys [n*k]: -1 stays -1,
 * an id outside [0, E) becomes -2 (still invalid for the E + r physical
 * experts), a valid id goes to the copy whose run holds its ordinal. */
void oracle_reroute(int64_t n, int k, int e, const int32_t *idx, int r, const int32_t *replica_of, int32_t *phys) {
  const int64_t a_n = n * k;
  int64_t *count = calloc((size_t)e, sizeof(int64_t)), *seen = calloc((size_t)e, sizeof(int64_t));
  for (int64_t a = 0; a < a_n; ++a)
    if (idx[a] >= 0 && idx[a] < e) ++count[idx[a]];
  for (int64_t a = 0; a < a_n; ++a) {
    const int32_t x = idx[a];
    if (x == -1) { phys[a] = -1; continue; }
    if (x < 0 || x >= e) { phys[a] = -2; continue; }
    int m = 1;
    for (int i = 0; i < r; ++i) m += replica_of[i] == x;
    const int64_t o = seen[x]++;
    int run = 0; /* the run whose ordinal range [ceil(j c/m), ceil((j+1) c/m)) holds o */
    while (!(o >= (run * count[x] + m - 1) / m && o < ((run + 1) * count[x] + m - 1) / m)) ++run;
    if (run == 0) { phys[a] = x; continue; }
    int slot = -1, found = 0; /* e's run-th slot, in slot order */
    for (int i = 0; i < r && found < run; ++i)
      if (replica_of[i] == x && ++found == run) slot = i;
    phys[a] = e + slot;
  }
  free(count);
  free(seen);
}

/* Replica weight sync: slot i's weights [elems] = its master's. */
void oracle_replica_sync(int r, const int32_t *replica_of, int64_t elems, const uint16_t *master, uint16_t *replica) {
  for (int i = 0; i < r; ++i)
    memcpy(replica + (int64_t)i * elems, master + (int64_t)replica_of[i] * elems, (size_t)elems * 2);
}

/* Replica gradient reduce: for every expert with slots, grad_master[e] =
 * bf16(grad_master[e] + the sum of its slots' gradients), the sum exact
 * (double; a handful of bf16 terms), one rounding. */
void oracle_replica_grad_reduce(int e, int r, const int32_t *replica_of, int64_t elems, const uint16_t *grad_replica,
                                uint16_t *grad_master) {
  for (int x = 0; x < e; ++x) {
    int any = 0;
    for (int i = 0; i < r; ++i) any |= replica_of[i] == x;
    if (!any) continue;
    for (int64_t v = 0; v < elems; ++v) {
      double acc = bf16_value(grad_master[(int64_t)x * elems + v]);
      for (int i = 0; i < r; ++i)
        if (replica_of[i] == x) acc += bf16_value(grad_replica[(int64_t)i * elems + v]);
      grad_master[(int64_t)x * elems + v] = bf16_round(acc);
    }
  }
}

/* ------------------------------------------------------------- expert FFN */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU expert [MEG experts(dispatched_input, tokens_per_expert, ...)], no bias.
 * For a row r in expert e's segment [offset_e, offset_e + kept_e):
 *   g_i = sum_h x[r,h] W_gu[e, i, h],  u_i = sum_h x[r,h] W_gu[e, I+i, h]
 *   a_i = bf16(silu(g_i) * u_i),       y[r,c] = bf16(sum_i a_i W_d[e, c, i])
 * with every sum in double (bf16 x bf16 products are exact in double).
 * Computes only the listed rows (y_rows[j] receives row rows[j]); a row outside
 * every segment is left untouched and reported by a -1 in expert_of. */
void oracle_expert_ffn_rows(int64_t nrows, const int64_t *rows, int e, int64_t h, int64_t inter,
                            const uint16_t *x_perm, const int32_t *expert_offsets,
                            const int32_t *tokens_per_expert, const uint16_t *w_gate_up,
                            const uint16_t *w_down, uint16_t *y_rows, int32_t *expert_of) {
  double *act = (double *)malloc(sizeof(double) * (size_t)inter);
  for (int64_t j = 0; j < nrows; ++j) {
    int64_t r = rows[j];
    int ex = -1;
    for (int x = 0; x < e; ++x)
      if (r >= expert_offsets[x] && r < (int64_t)expert_offsets[x] + tokens_per_expert[x]) { ex = x; break; }
    if (expert_of) expert_of[j] = ex;
    if (ex < 0) continue;
    const uint16_t *xr = x_perm + r * h;
    const uint16_t *wg = w_gate_up + (int64_t)ex * 2 * inter * h;
    const uint16_t *wd = w_down + (int64_t)ex * h * inter;
    for (int64_t i = 0; i < inter; ++i) {
      double g = 0.0, u = 0.0;
      for (int64_t c = 0; c < h; ++c) {
        double xv = bf16_value(xr[c]);
        g += xv * bf16_value(wg[i * h + c]);
        u += xv * bf16_value(wg[(inter + i) * h + c]);
      }
      act[i] = bf16_value(bf16_round(silu(g) * u));
    }
    for (int64_t c = 0; c < h; ++c) {
      double s = 0.0;
      for (int64_t i = 0; i < inter; ++i) s += act[i] * bf16_value(wd[c * inter + i]);
      y_rows[j * h + c] = bf16_round(s);
    }
  }
  free(act);
}

/* ----------------------------------------------------------------- combine */

/* Probability-weighted combine [DS restore_combined: weighted rows are added by
 * token index into a zeroed output one top-k slot at a time; MEG
 * combine_postprocess].  out[t,h] = sum over kept slots j = 0..k-1, in that
 * order, of topk_w[t,j] * y[assign_row[t,j], h], accumulated in fp32 with a
 * fused multiply-add per term (C99 fmaf is correctly rounded), then rounded once
 * to the output type.  A token with no kept slot gets a zero row. */
void oracle_combine(int64_t n, int k, int64_t h, int dt, const void *y, const float *topk_w,
                    const int32_t *assign_row, void *out) {
  for (int64_t t = 0; t < n; ++t) {
    for (int64_t c = 0; c < h; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        int32_t r = assign_row[t * k + j];
        if (r < 0) continue;
        acc = fmaf(topk_w[t * k + j], (float)act_load(y, dt, (int64_t)r * h + c), acc);
      }
      act_store(out, dt, t * h + c, (double)acc);
    }
  }
}

/* Dispatch backward: the vector-Jacobian product of the row scatter (dispatch
 * copies token t's row to the rows of its kept slots; the MORI pull request
 * ROCm/Megatron-LM "Add MORI as a Token Dispatcher" lists the unpermute /
 * dispatch backward among the paths it fixes).  For each token t:
 *   grad_x[t, :] = sum over kept slots j, in slot order, of grad_x_perm[assign_row[t,j], :]
 * fp32 accumulation, one rounding to the activation type; a token with no kept
 * slot gets a zero row. */
void oracle_dispatch_bwd(int64_t n, int k, int64_t h, int dt, const void *grad_x_perm, const int32_t *assign_row,
                         void *grad_x) {
  for (int64_t t = 0; t < n; ++t) {
    for (int64_t c = 0; c < h; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        int32_t r = assign_row[t * k + j];
        if (r < 0) continue;
        acc = acc + (float)act_load(grad_x_perm, dt, (int64_t)r * h + c);
      }
      act_store(grad_x, dt, t * h + c, (double)acc);
    }
  }
}

/* Combine backward (the vector-Jacobian product of the combine above; the MORI
 * commit log's combine backward takes the receiver-side weights and indices).
 * For each kept assignment a = (t, j) in row r:
 *   grad_y[r, :] = w[t,j] * g[t, :]        (one rounding to the activation type)
 *   grad_w[t, j] = sum_h g[t,h] * y[r,h]   (double, one rounding to fp32)
 * grad_w is 0 for dropped, sentinel and invalid slots; pad rows of grad_y
 * (rows below pad_limit holding no assignment) are 0; rows of an unused
 * dropless tail are not written. */
void oracle_combine_bwd(int64_t n, int k, int64_t h, int dt, const void *grad_out, const void *y,
                        const float *topk_w, const int32_t *assign_row, int64_t rows,
                        const int32_t *row_src, int64_t pad_limit, void *grad_y, float *grad_w) {
  for (int64_t t = 0; t < n; ++t) {
    for (int j = 0; j < k; ++j) {
      int64_t a = t * k + j;
      int32_t r = assign_row[a];
      if (r < 0) { grad_w[a] = 0.0f; continue; }
      double dot = 0.0;
      for (int64_t c = 0; c < h; ++c) {
        double g = act_load(grad_out, dt, t * h + c);
        dot += g * act_load(y, dt, (int64_t)r * h + c);
        act_store(grad_y, dt, (int64_t)r * h + c, (double)topk_w[a] * g);
      }
      grad_w[a] = (float)dot;
    }
  }
  for (int64_t r = 0; r < rows && r < pad_limit; ++r)
      if (row_src[r] < 0)
        for (int64_t c = 0; c < h; ++c) act_store(grad_y, dt, r * h + c, 0.0);
}

/* Exposed for the tests that pin the number formats. */
uint16_t oracle_bf16_round(double x) { return bf16_round(x); }

/* Element-wise double -> bf16 (round to nearest, ties to even) of n values. */
void oracle_bf16_round_array(int64_t n, const double *x, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(x[i]);
}
