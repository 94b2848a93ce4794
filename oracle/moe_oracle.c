/*
 * CPU oracle for the MXFP4 MoE expert layer -- TEST INFRASTRUCTURE.
 *
 * Plain, slow, fp64 reference of what the layer computes.  Only the tests, the
 * package's smoke check and the benchmark's CPU-baseline leg may build, load
 * or run this file.  It shares no code, header, table or helper with the GPU
 * library: both consume the same input bytes and nothing else.
 *
 * Sources (each function names the passage it follows):
 *  [P1-FP4]  page "MiMo x TileRT" article on blog.hypho.cn (tags/speculative-
 *            decoding), section "第一层：FP4 选择性量化": the MoE experts are
 *            stored in OCP MXFP4 while the router keeps a higher precision.
 *  [P1-BG]   same page, section "万亿参数推理为什么特别难": MoE routes each
 *            token to a few experts; decode is bound by the bytes read.
 *  [P3-FP4]  page "MiMo 把 1T 模型推到每秒千 token——FP4、DFlash 與常駐 kernel
 *            的三層 co-design" (vatt-ghern.pages.dev), section "FP4：只量化 MoE
 *            expert，其餘維持原精度": weights are cut into small blocks, each
 *            block stores 4-bit values plus one shared higher-precision scale;
 *            the router's top-k choice is precision sensitive.
 *  [P5-FP4]  page "tech-implementation-2026-06-09" (shengyayun.com), section
 *            "关键实现细节 / 1. 为什么是 FP4 量化 + 只量化 MoE Experts": the
 *            quantized linears are the experts' gate_proj, up_proj, down_proj.
 *  [P5-TRT]  same page, section "3. TileRT 的"持久化内核"到底做了什么": per
 *            layer the forward runs the MoE gate, then the expert compute.
 *  [MX]      the OCP Microscaling Formats (MX) v1.0 specification that pages 1
 *            and 5 list among their sources: FP4 elements are E2M1 (1 sign,
 *            2 exponent bits with bias 1, 1 mantissa bit, no inf/NaN), a block
 *            is 32 elements, the shared scale is E8M0 (2^(s-127), s=255 NaN).
 *
 * Readings where the pages are silent (also listed in the design notes):
 *  - storage: rows of K elements, row-major, K the reduction dimension;
 *    element c in byte c/2 of its row, low nibble for even c; one scale byte
 *    per 32 consecutive elements of a row;
 *  - expert e's bytes are contiguous: gate [F][d] | up [F][d] | down [d][F],
 *    scales likewise (gate [F][d/32] | up [F][d/32] | down [d][F/32]);
 *  - expert FFN: h = silu(gate x) * (up x), y = down h, silu(z) = z/(1+e^-z);
 *  - top-k: the k largest logits, ties broken toward the lower expert index;
 *    gates: softmax over the k selected logits (equal to a full softmax
 *    renormalised over the selected set);
 *  - permutation: (token, expert) pairs ordered by expert, then token;
 *  - output: out[t] = sum over the token's k slots j (in top-k order) of
 *    gate[t][j] * y(expert_j, t).
 *
 * Parity pins: every function is checked by the CPU tests against closed
 * forms, invariants and an independent dense brute-force evaluation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- format --- */

/* E2M1 code -> value.  [MX]: bit 3 sign, bits 2..1 exponent E (bias 1),
 * bit 0 mantissa M; E == 0 is subnormal: M * 0.5; otherwise 2^(E-1)*(1+M/2). */
double oracle_e2m1(unsigned code) {
  unsigned s = (code >> 3) & 1u, E = (code >> 1) & 3u, M = code & 1u;
  double mag = (E == 0) ? 0.5 * (double)M : ldexp(1.0 + 0.5 * (double)M, (int)E - 1);
  return s ? -mag : mag;
}

/* E8M0 scale byte -> value.  [MX]: 2^(s-127); s = 255 encodes NaN. */
double oracle_e8m0(unsigned s) {
  if (s == 255u) return NAN;
  return ldexp(1.0, (int)s - 127);
}

/* bf16 bit pattern -> value (bf16 is the top half of an IEEE binary32). */
double oracle_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Element (r, c) of a stored MXFP4 matrix with K columns. [P3-FP4], [MX]:
 * the 4-bit value times the scale of its 32-element block. */
double oracle_mxfp4_element(const uint8_t* P, const uint8_t* S, int64_t K, int64_t r, int64_t c) {
  uint8_t byte = P[r * (K / 2) + c / 2];
  unsigned code = (c % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
  return oracle_e2m1(code) * oracle_e8m0(S[r * (K / 32) + c / 32]);
}

/* out[r][c] for all rows and columns (exact in fp64). */
void oracle_dequantize(const uint8_t* P, const uint8_t* S, int64_t rows, int64_t K, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < K; ++c) out[r * K + c] = oracle_mxfp4_element(P, S, K, r, c);
}

/* Quantize rows of doubles to MXFP4 ([P3-FP4] "4-bit values + per-block
 * scale"; [MX] conversion): shared exponent X = floor(log2 amax) - 2 (the
 * largest E2M1 exponent is 2), clamped to [-127, 127], X = -127 for an
 * all-zero block; each element v/2^X goes to the nearest E2M1 magnitude,
 * ties to the one with an even mantissa bit, saturating at 6; the sign bit is
 * set when v < 0.  Written here only to pin the format (round trips). */
void oracle_quantize(const double* w, int64_t rows, int64_t K, uint8_t* P, uint8_t* S) {
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < K / 32; ++b) {
      const double* v = w + r * K + b * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
      int X = -127;
      if (amax > 0.0) {
        X = (int)floor(log2(amax)) - 2;
        /* guard log2 rounding at exact powers of two */
        while (ldexp(1.0, X + 2) > amax) --X;
        while (ldexp(1.0, X + 3) <= amax) ++X;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
      }
      S[r * (K / 32) + b] = (uint8_t)(X + 127);
      for (int i = 0; i < 32; ++i) {
        double q = fabs(v[i]) / ldexp(1.0, X);
        unsigned best = 0;
        double bestd = INFINITY;
        for (unsigned m = 0; m < 8; ++m) {
          double dist = fabs(q - oracle_e2m1(m));
          if (dist < bestd || (dist == bestd && (m & 1u) == 0)) {
            bestd = dist;
            best = m;
          }
        }
        if (q > 6.0) best = 7;
        unsigned code = best | (v[i] < 0.0 ? 8u : 0u);
        int64_t c = b * 32 + i;
        uint8_t* byte = &P[r * (K / 2) + c / 2];
        if (c % 2 == 0)
          *byte = (uint8_t)((*byte & 0xF0u) | code);
        else
          *byte = (uint8_t)((*byte & 0x0Fu) | (code << 4));
      }
    }
  }
}

/* ---------------------------------------------------------------- router --- */

/* logits[t][e] = sum_c x[t][c] * W_r[e][c] in fp64.  [P1-FP4], [P3-FP4]: the
 * router stays at higher precision than the experts (fp32 weights here). */
void oracle_router(const uint16_t* x, const float* wr, int T, int d, int E, double* logits) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += oracle_bf16(x[(int64_t)t * d + c]) * (double)wr[(int64_t)e * d + c];
      logits[(int64_t)t * E + e] = acc;
    }
}

/* Order used for top-k: larger logit first, then lower expert index. */
static const double* g_sort_row;
static int cmp_logit_desc(const void* a, const void* b) {
  int ia = *(const int*)a, ib = *(const int*)b;
  double la = g_sort_row[ia], lb = g_sort_row[ib];
  if (la > lb) return -1;
  if (la < lb) return 1;
  return (ia > ib) - (ia < ib);
}

/* Per token: the k experts with the largest logits ([P1-BG] a token is sent
 * to a few experts; [P3-FP4] top-k selection), in (logit desc, index asc)
 * order, and their gates: softmax over the k selected logits (max
 * subtracted).  Returns the smallest gap l_(k) - l_(k+1) over all tokens
 * (+inf when k == E), which tells whether the selection is well separated. */
double oracle_topk(const double* logits, int T, int E, int k, int32_t* idx, double* gates) {
  int* order = (int*)malloc(sizeof(int) * (size_t)E);
  double min_gap = INFINITY;
  for (int t = 0; t < T; ++t) {
    const double* row = logits + (int64_t)t * E;
    for (int e = 0; e < E; ++e) order[e] = e;
    g_sort_row = row;
    qsort(order, (size_t)E, sizeof(int), cmp_logit_desc);
    double lmax = row[order[0]];
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += exp(row[order[j]] - lmax);
    for (int j = 0; j < k; ++j) {
      idx[(int64_t)t * k + j] = order[j];
      gates[(int64_t)t * k + j] = exp(row[order[j]] - lmax) / z;
    }
    if (k < E) {
      double gap = row[order[k - 1]] - row[order[k]];
      if (gap < min_gap) min_gap = gap;
    }
  }
  free(order);
  return min_gap;
}

/* ------------------------------------------------------------- permutation --- */

/* Token-to-expert permutation: the T*k (token, slot) pairs ordered by expert,
 * then by token.  offsets[e] = number of pairs with expert < e (E+1 entries),
 * sorted_slot[p] = t*k + j of the p-th pair, pos[t*k + j] = p.
 * [P1-BG] each expert processes the tokens routed to it. */
void oracle_permute(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* sorted_slot,
                    int32_t* pos) {
  int32_t* count = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int64_t s = 0; s < (int64_t)T * k; ++s) count[idx[s]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + count[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int t = 0; t < T; ++t)       /* tokens in ascending order ...            */
    for (int j = 0; j < k; ++j) {   /* ... so each expert's list is token-sorted */
      int e = idx[(int64_t)t * k + j];
      int32_t p = fill[e]++;
      sorted_slot[p] = t * k + j;
      pos[(int64_t)t * k + j] = p;
    }
  free(count);
  free(fill);
}

/* ---------------------------------------------------------------- experts --- */

/* silu(z) = z * sigmoid(z). */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Expert e applied to the tokens of pairs [p0, p1): [P5-FP4] gate_proj,
 * up_proj and down_proj are the expert's MXFP4 linears; the activation
 * between them is SwiGLU: h = silu(W_gate x) * (W_up x), y = W_down h.
 * Hot loop: decode one weight row to fp64, then dot it with every token.
 * h: [pairs][F] (pair order), y: [pairs][d]. */
static void expert_apply(const uint8_t* pk, const uint8_t* sc, int d, int F, const double* xd,
                         const int32_t* sorted_slot, int k, const uint8_t* token_mask, int32_t p0,
                         int32_t p1, double* h, double* y) {
  const uint8_t* pg = pk;
  const uint8_t* pu = pk + (int64_t)F * d / 2;
  const uint8_t* pdn = pk + (int64_t)F * d;
  const uint8_t* sg = sc;
  const uint8_t* su = sc + (int64_t)F * d / 32;
  const uint8_t* sdn = sc + (int64_t)F * d / 16;
  double* rowg = (double*)malloc(sizeof(double) * (size_t)d);
  double* rowu = (double*)malloc(sizeof(double) * (size_t)d);
  double* rowd = (double*)malloc(sizeof(double) * (size_t)F);
  for (int i = 0; i < F; ++i) {
    oracle_dequantize(pg + (int64_t)i * d / 2, sg + (int64_t)i * d / 32, 1, d, rowg);
    oracle_dequantize(pu + (int64_t)i * d / 2, su + (int64_t)i * d / 32, 1, d, rowu);
    for (int32_t p = p0; p < p1; ++p) {
      int t = sorted_slot[p] / k;
      if (token_mask && !token_mask[t]) continue;
      const double* xt = xd + (int64_t)t * d;
      double g = 0.0, u = 0.0;
      for (int c = 0; c < d; ++c) {
        g += rowg[c] * xt[c];
        u += rowu[c] * xt[c];
      }
      h[(int64_t)p * F + i] = oracle_silu(g) * u;
    }
  }
  for (int r = 0; r < d; ++r) {
    oracle_dequantize(pdn + (int64_t)r * F / 2, sdn + (int64_t)r * F / 32, 1, F, rowd);
    for (int32_t p = p0; p < p1; ++p) {
      int t = sorted_slot[p] / k;
      if (token_mask && !token_mask[t]) continue;
      const double* hp = h + (int64_t)p * F;
      double acc = 0.0;
      for (int i = 0; i < F; ++i) acc += rowd[i] * hp[i];
      y[(int64_t)p * d + r] = acc;
    }
  }
  free(rowg);
  free(rowu);
  free(rowd);
}

/* ---------------------------------------------------------------- layer --- */

/* One MoE layer ([P5-TRT]: MoE gate, then expert compute; the combine weights
 * each expert's output by its gate).  Inputs: x bf16 [T][d], W_r fp32 [E][d],
 * packed/scales as described in the header, top-k k.  token_mask (may be
 * NULL) restricts the expert FFN and combine to the marked tokens; routing is
 * always computed for all tokens.  Optional outputs may be NULL:
 *   logits [T][E], idx [T][k], gates [T][k], offsets [E+1], sorted_slot [T*k],
 *   pos [T*k], h [T*k][F] (pair order), y [T*k][d] (pair order, no gate).
 * out [T][d] (rows of unmasked tokens are left untouched).
 * Returns the smallest top-k gap, or NaN on bad arguments / allocation. */
double oracle_forward(int T, int d, int F, int E, int k, const uint16_t* x, const float* wr,
                      const uint8_t* packed, const uint8_t* scales, const uint8_t* token_mask,
                      int nthreads, double* out, double* logits_o, int32_t* idx_o, double* gates_o,
                      int32_t* offsets_o, int32_t* sorted_slot_o, int32_t* pos_o, double* h_o,
                      double* y_o) {
  if (T < 0 || d <= 0 || F <= 0 || E <= 0 || k < 1 || k > E || d % 32 || F % 32) return NAN;
  if (T == 0) return INFINITY;
  const int64_t TK = (int64_t)T * k;
  double* xd = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* logits = logits_o ? logits_o : (double*)malloc(sizeof(double) * (size_t)T * E);
  int32_t* idx = idx_o ? idx_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)TK);
  double* gates = gates_o ? gates_o : (double*)malloc(sizeof(double) * (size_t)TK);
  int32_t* offsets = offsets_o ? offsets_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
  int32_t* sslot = sorted_slot_o ? sorted_slot_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)TK);
  int32_t* pos = pos_o ? pos_o : (int32_t*)malloc(sizeof(int32_t) * (size_t)TK);
  double* h = h_o ? h_o : (double*)calloc((size_t)TK * F, sizeof(double));
  double* y = y_o ? y_o : (double*)calloc((size_t)TK * d, sizeof(double));
  if (!xd || !logits || !idx || !gates || !offsets || !sslot || !pos || !h || !y) return NAN;

  for (int64_t i = 0; i < (int64_t)T * d; ++i) xd[i] = oracle_bf16(x[i]);
  oracle_router(x, wr, T, d, E, logits);
  double gap = oracle_topk(logits, T, E, k, idx, gates);
  oracle_permute(idx, T, E, k, offsets, sslot, pos);

  const int64_t pbytes = (int64_t)3 * d * F / 2, sbytes = (int64_t)3 * d * F / 32;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int e = 0; e < E; ++e) {
    int used = 0; /* skip experts none of whose tokens is requested */
    for (int32_t p = offsets[e]; p < offsets[e + 1] && !used; ++p)
      used = !token_mask || token_mask[sslot[p] / k];
    if (!used) continue;
    expert_apply(packed + e * pbytes, scales + e * sbytes, d, F, xd, sslot, k, token_mask,
                 offsets[e], offsets[e + 1], h, y);
  }
  (void)nthreads;

  for (int t = 0; t < T; ++t) {
    if (token_mask && !token_mask[t]) continue;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += gates[(int64_t)t * k + j] * y[(int64_t)pos[(int64_t)t * k + j] * d + c];
      out[(int64_t)t * d + c] = acc;
    }
  }

  free(xd);
  if (!logits_o) free(logits);
  if (!idx_o) free(idx);
  if (!gates_o) free(gates);
  if (!offsets_o) free(offsets);
  if (!sorted_slot_o) free(sslot);
  if (!pos_o) free(pos);
  if (!h_o) free(h);
  if (!y_o) free(y);
  return gap;
}
