/*
 * hsa_oracle.c -- plain, slow CPU reference for Hierarchical Sparse Attention (HSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file; it exists so that tests, the smoke check and the CPU-baseline leg of the
 * benchmark can compare the GPU library against an independent definition.  It shares
 * no code, header, table or helper with the HIP library.
 *
 * Everything is computed in IEEE double from the stored input values (fp32 or bf16,
 * both exactly representable in double), with plain loops in the order the method
 * states its steps.  OpenMP only splits independent rows; it never changes an
 * arithmetic order.
 *
 * Sources (the pages describing the method):
 *   [HSA-note]  "Hardware-aligned Hierarchical Sparse Attention for Efficient Long-term
 *               Memory Access", papernotes.org NeurIPS 2025 note, section 方法详解:
 *               subsections 整体架构（RAMba）, 层次化稀疏注意力（HSA）, 硬件对齐 Kernel,
 *               训练与推理优化.
 *   [HSA-atlas] same paper, atlas.scime.ai summary, section "Approach".
 *   [HSA-abs]   same paper, paperdance.org abstract.
 *
 * Readings where the pages are silent (each one is also listed with the design notes):
 *   - softmax-off-by-one = softmax with one extra logit fixed at 0 whose value row is 0:
 *       a_j = exp(z_j) / (1 + sum_i exp(z_i)).
 *   - token-level logits are scaled by sm_scale (1/sqrt(d) by default); selection scores
 *     are sel_scale * <Qs, Kslc> (1/sqrt(d) by default).
 *   - token t may select chunk c only if c < floor(t/S); fewer than K candidates leave the
 *     remaining slots masked (idx -1, score -inf, weight 0).
 *   - ranking is by score descending, ties toward the lower chunk index; stick-breaking
 *     runs over the slots in that rank order; a NaN score ranks as -inf.
 *   - the softmax variant of the chunk weights is a plain softmax of the valid slots'
 *     selection scores (no temperature), masked slots 0.
 *   - the chunk key is the plain mean of the chunk's S key rows, rounded once (to nearest,
 *     ties to even) to the storage type of the inputs; selection scores are rounded to fp32
 *     before ranking, the precision in which the GPU library takes the same decision.
 *   - query head h belongs to KV group floor(h / (Hq/Hkv)).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Compile-time switch used only by the oracle's own self-tests: a nonzero value plants
 * one known mistake so the tests can show that some pin catches it.  0 = the oracle. */
#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif
#define MUT(n) (ORACLE_MUTATION == (n))

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

/* Threads of the OpenMP row loops from now on (timing aid; no arithmetic depends on it). */
void oracle_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int oracle_max_threads(void) { return omp_get_max_threads(); }

/* ---- storage helpers ------------------------------------------------------------- */

/* Read element i of an fp32 or bf16 array as a double (exact). */
static double ld(const void* p, size_t i, int dt) {
  if (dt == ORC_BF16) {
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  if (dt == ORC_F64) return ((const double*)p)[i];
  return (double)((const float*)p)[i];
}

/* Round x to the nearest value of storage type dt, ties to even.
 * bf16 has 8 significant bits and fp32's exponent range; its subnormal spacing is 2^-133. */
double oracle_round(double x, int dt) {
  if (dt == ORC_F32) return (double)(float)x; /* C conversion: round to nearest even */
  if (dt != ORC_BF16) return x;
  if (x == 0.0 || !isfinite(x)) return x;
  double a = fabs(x);
  int e = ilogb(a);            /* a = m * 2^e with 1 <= m < 2 */
  if (e < -126) e = -126;      /* below the normal range the spacing stops shrinking */
  int q = e - 7;               /* spacing of bf16 values near a */
  double r = nearbyint(ldexp(a, -q)); /* default rounding mode: nearest, ties to even */
  double y = ldexp(r, q);
  if (y > 3.3895313892515355e38) y = INFINITY; /* beyond the largest finite bf16 */
  return x < 0 ? -y : y;
}

/* ---- F1: chunk keys by mean pooling ------------------------------------------------
 * [HSA-note 层次化稀疏注意力（HSA）, "Chunk Selection"]: a chunk is represented by the mean
 * of its keys; [HSA-note 训练与推理优化, "KV Cache Offloading"]: the chunk table has
 * floor(L/S) rows of width d per group.
 * K: [B, L, Hkv, D] (dtype dt).  Kslc out: [B, nC, Hkv, D] double, rounded to round_dt. */
void oracle_pool(const void* K, int dt, int B, int L, int Hkv, int D, int S, int round_dt,
                 double* Kslc) {
  int nC = L / S;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < nC; ++c)
      for (int g = 0; g < Hkv; ++g)
        for (int e = 0; e < D; ++e) {
          double sum = 0.0;
          int rows = MUT(5) ? S - 1 : S;
          for (int j = 0; j < rows; ++j)
            sum += ld(K, (((size_t)b * L + (size_t)c * S + j) * Hkv + g) * D + e, dt);
          double mean = sum / S;
          Kslc[(((size_t)b * nC + c) * Hkv + g) * D + e] = oracle_round(mean, round_dt);
        }
}

/* ---- F2-F4: per-query-group top-K selection and stick-breaking weights ------------ */

typedef struct { double s; int c; } cand_t;

/* Rank order: higher score first; equal scores -> lower chunk index first. */
static int cand_cmp(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  if (MUT(3)) return (a->c < b->c) ? 1 : (a->c > b->c) ? -1 : 0;
  return (a->c < b->c) ? -1 : (a->c > b->c) ? 1 : 0;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Stick-breaking over the valid slots in rank order:
 * w_k = sigma(s_k) * prod_{j<k} (1 - sigma(s_j))
 * [HSA-note 层次化稀疏注意力（HSA）, 第二阶段: weights depend only on the sigmoid of the
 * relevance scores and carry no positional encoding]. */
static void stick_breaking(const double* s, int n_valid, double* w) {
  double remaining = 1.0;
  for (int k = 0; k < n_valid; ++k) {
    double p = sigmoid(s[k]);
    w[k] = p * remaining;
    remaining *= MUT(2) ? p : (1.0 - p);
  }
}

/* The softmax variant of the chunk weights: w_k = exp(s_k) / sum_j exp(s_j) over the valid
 * slots, evaluated with the shift m = max_j s_j (all weights 0 if every score is -inf)
 * [HSA-atlas, "Measured effects reported in the paper": the ablation that replaces the
 * stick-breaking weights with a softmax; HSA-note 亮点: softmax vs stick-breaking]. */
enum { ORC_W_STICK = 0, ORC_W_SOFTMAX = 1 };
static void softmax_weights(const double* s, int n_valid, double* w) {
  double m = -INFINITY;
  for (int k = 0; k < n_valid; ++k)
    if (s[k] > m) m = s[k];
  double den = 0.0;
  for (int k = 0; k < n_valid; ++k) {
    w[k] = m == -INFINITY ? 0.0 : exp(s[k] - m);
    den += w[k];
  }
  for (int k = 0; k < n_valid; ++k) w[k] = den > 0.0 ? w[k] / den : 0.0;
}

/* Number of chunks token t may select (causal: strictly earlier, complete chunks). */
static int n_available(int t, int S, int nC) {
  int n = MUT(4) ? t / S + 1 : t / S;
  return n < nC ? n : nC;
}

/* Selection score of (query row qs, chunk key row) rounded to the score precision. */
static double sel_score(const void* Qs, int dt, size_t qoff, const double* krow, int D,
                        double sel_scale, int score_dt) {
  double dot = 0.0;
  for (int e = 0; e < D; ++e) dot += ld(Qs, qoff + e, dt) * krow[e];
  double s = oracle_round(sel_scale * dot, score_dt);
  if (isnan(s) && !MUT(12)) s = -INFINITY; /* a NaN score ranks last and carries no weight */
  return s;
}

/* Fill one row's K slots from an array of scored candidates. */
static void select_row(cand_t* cand, int n_avail, int Kt, int wmode, int32_t* idx,
                       double* score, double* w) {
  qsort(cand, (size_t)n_avail, sizeof(cand_t), cand_cmp);
  int n_valid = n_avail < Kt ? n_avail : Kt;
  double sv[64];
  for (int k = 0; k < n_valid; ++k) {
    idx[k] = cand[k].c;
    score[k] = cand[k].s;
    sv[k] = cand[k].s;
  }
  double wv[64];
  if (wmode == ORC_W_SOFTMAX)
    softmax_weights(sv, n_valid, wv);
  else
    stick_breaking(sv, n_valid, wv);
  for (int k = 0; k < Kt; ++k) {
    if (k < n_valid) {
      w[k] = wv[k];
    } else {
      idx[k] = -1;
      score[k] = -INFINITY;
      w[k] = 0.0;
    }
  }
}

/* Qs: [B, L, Hkv, D]; Kslc: [B, nC, Hkv, D] double (from oracle_pool).
 * Out idx/score/w: [B, L, Hkv, Kt].  row_mask (optional, [B*L]): rows with 0 are skipped.
 * [HSA-note 层次化稀疏注意力（HSA）, "Chunk Selection"]: every token scores each chunk's
 * pooled key with its selection query and keeps the top-K, separately per query group. */
void oracle_select(const void* Qs, int dt, const double* Kslc, int B, int L, int Hkv, int D,
                   int S, int Kt, double sel_scale, int score_dt, int wmode,
                   const uint8_t* row_mask, int32_t* idx, double* score, double* w) {
  int nC = L / S;
#pragma omp parallel
  {
    cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(nC > 0 ? nC : 1));
#pragma omp for collapse(2) schedule(dynamic, 64)
    for (int b = 0; b < B; ++b)
      for (int t = 0; t < L; ++t) {
        if (row_mask && !row_mask[(size_t)b * L + t]) continue;
        int n_avail = n_available(t, S, nC);
        for (int g = 0; g < Hkv; ++g) {
          size_t qoff = (((size_t)b * L + t) * Hkv + g) * D;
          for (int c = 0; c < n_avail; ++c) {
            const double* krow = Kslc + (((size_t)b * nC + c) * Hkv + g) * D;
            cand[c].s = sel_score(Qs, dt, qoff, krow, D, sel_scale, score_dt);
            cand[c].c = c;
          }
          size_t o = (((size_t)b * L + t) * Hkv + g) * Kt;
          select_row(cand, n_avail, Kt, wmode, idx + o, score + o, w + o);
        }
      }
    free(cand);
  }
}

/* ---- F5: softmax-off-by-one attention inside one chunk -----------------------------
 * [HSA-note 层次化稀疏注意力（HSA）, 第一阶段]: ordinary attention of the token's query over
 * the S keys of one selected chunk; [HSA-note 硬件对齐 Kernel]: normalised with
 * softmax-off-by-one so that a token can give the chunk little total weight.
 * z_j = sm_scale <q, k_j>;  a_j = exp(z_j) / (1 + sum_i exp(z_i)), evaluated with the
 * shift m = max(0, max_j z_j) so no exponential overflows.
 * a: out [S] probabilities; returns the normaliser's log, log(1 + sum_j exp(z_j)) =
 * m + log(exp(-m) + sum_j exp(z_j - m)). */
static double softmax1_probs(const void* Q, int dtq, size_t qoff, const void* K, int dtk,
                           size_t k0, size_t kstride, int D, int S, double sm_scale,
                           double* a) {
  double z[1024];
  double m = 0.0;
  for (int j = 0; j < S; ++j) {
    double dot = 0.0;
    for (int e = 0; e < D; ++e) dot += ld(Q, qoff + e, dtq) * ld(K, k0 + j * kstride + e, dtk);
    z[j] = MUT(10) ? dot : sm_scale * dot;
    if (z[j] > m) m = z[j];
  }
  double den = MUT(1) ? 0.0 : exp(-m); /* the extra zero logit */
  for (int j = 0; j < S; ++j) {
    a[j] = exp(z[j] - m);
    den += a[j];
  }
  for (int j = 0; j < S; ++j) a[j] /= den;
  return m + log(den);
}

/* Query head h -> KV group. */
static int group_of(int h, int Hq, int Hkv) {
  if (MUT(9)) return h % Hkv;
  return h / (Hq / Hkv);
}

/* ---- F5-F6: token-level attention fused with the chunk weights ---------------------
 * [HSA-note 层次化稀疏注意力（HSA）, 第二阶段] and [HSA-note 硬件对齐 Kernel, forward]:
 * O_t = sum_k w_k * O_{t,k}; a token with no valid slot gets O_t = 0.
 * Q: [B, L, Hq, D]; K, V: [B, L, Hkv, D]; idx/w: [B, L, Hkv, Kt].  O out: [B, L, Hq, D].
 * Ok (optional): per-slot unweighted outputs [B, L, Hq, Kt, D] (0 for masked slots).
 * lse (optional): per (token, head, slot) the normaliser's log, log(1 + sum_j exp(z_j)),
 * [B, L, Hq, Kt] (0 for masked slots). */
void oracle_attend(const void* Q, const void* K, const void* V, int dt, const int32_t* idx,
                   const double* w, int B, int L, int Hq, int Hkv, int D, int S, int Kt,
                   double sm_scale, const uint8_t* row_mask, double* O, double* Ok,
                   double* lse) {
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < L; ++t) {
      if (row_mask && !row_mask[(size_t)b * L + t]) continue;
      double a[1024];
      for (int h = 0; h < Hq; ++h) {
        int g = group_of(h, Hq, Hkv);
        size_t qoff = (((size_t)b * L + t) * Hq + h) * D;
        double* out = O + qoff;
        for (int e = 0; e < D; ++e) out[e] = 0.0;
        for (int k = 0; k < Kt; ++k) {
          size_t so = (((size_t)b * L + t) * Hkv + g) * Kt + k;
          int c = idx[so];
          double* ok = Ok ? Ok + ((((size_t)b * L + t) * Hq + h) * Kt + k) * D : NULL;
          double* lk = lse ? lse + (((size_t)b * L + t) * Hq + h) * Kt + k : NULL;
          if (ok)
            for (int e = 0; e < D; ++e) ok[e] = 0.0;
          if (lk) *lk = 0.0;
          if (c < 0) continue;
          size_t k0 = (((size_t)b * L + (size_t)c * S) * Hkv + g) * D;
          size_t kstride = (size_t)Hkv * D;
          double lz = softmax1_probs(Q, dt, qoff, K, dt, k0, kstride, D, S, sm_scale, a);
          if (lk) *lk = lz;
          for (int e = 0; e < D; ++e) {
            double acc = 0.0;
            for (int j = 0; j < S; ++j) acc += a[j] * ld(V, k0 + j * kstride + e, dt);
            if (ok) ok[e] = acc;
            out[e] += w[so] * acc;
          }
        }
      }
    }
}

/* ---- B1-B5: backward with the selection fixed ----------------------------------------
 * [HSA-note 硬件对齐 Kernel]: the backward runs in two phases, first the gradients of the
 * queries and chunk weights per token, then the gradients of keys and values per chunk
 * over every token that selected it.  [HSA-note 层次化稀疏注意力（HSA）, 端到端学习] and
 * [HSA-atlas Approach]: the chunk weights pass gradient back into the selection scores.
 *
 * For token t, group g, valid slot k (chunk c, weight w_k, p_k = sigmoid(s_k)), head h:
 *   dA'_j = <dO_h, v_j>,  D_hk = sum_j a_j dA'_j,  dz_j = w_k a_j (dA'_j - D_hk)
 *   dQ_h += sm_scale sum_j dz_j k_j;   dK_j += sm_scale dz_j q_h;   dV_j += w_k a_j dO_h
 *   dw_k = sum_{h in g} D_hk
 *   ds_k = dw_k w_k (1 - p_k) - p_k sum_{k'>k} dw_{k'} w_{k'}   (stick-breaking chain rule)
 *   ds_k = w_k (dw_k - sum_j w_j dw_j)                           (softmax weights, wmode 1)
 *   dQs += sel_scale ds_k Kslc_c;  dKslc_c += sel_scale ds_k Qs_t
 * With fold != 0 the pooled-key gradient flows on into the keys: dK_j += dKslc_c / S for
 * every row j of chunk c (the chunk key is the mean of those rows).
 *
 * Inputs: Q [B,L,Hq,D], K, V, Qs [B,L,Hkv,D] (dtype dt); Kslc [B,nC,Hkv,D] double;
 *         idx/score/w [B,L,Hkv,Kt]; dO [B,L,Hq,D] (dtype dt).
 * Outputs (double): dQ [B,L,Hq,D], dK, dV, dQs [B,L,Hkv,D], dKslc [B,nC,Hkv,D],
 *         dw, ds [B,L,Hkv,Kt].
 * tok_mask [B*L] (optional) limits phase 1 (dQ, dQs, written rows only);
 * chunk_mask [B*nC] (optional) limits phase 2 (dK, dV, dKslc of those chunks only).
 * Phase 2 always needs ds of every token, so phase 1's ds is computed for all rows. */
void oracle_bwd(const void* Q, const void* K, const void* V, const void* Qs, int dt,
                const double* Kslc, const int32_t* idx, const double* score,
                const double* w, const void* dO, int B, int L, int Hq, int Hkv, int D, int S,
                int Kt, double sm_scale, double sel_scale, int fold, int wmode,
                const uint8_t* tok_mask, const uint8_t* chunk_mask, double* dQ, double* dK,
                double* dV, double* dQs, double* dKslc, double* dw, double* ds) {
  int nC = L / S;
  int G = Hq / Hkv;
  size_t kstride = (size_t)Hkv * D;

  /* Phase 1: per token and group. */
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < L; ++t) {
      int want_q = !tok_mask || tok_mask[(size_t)b * L + t];
      double a[1024], dA[1024];
      for (int g = 0; g < Hkv; ++g) {
        size_t so = (((size_t)b * L + t) * Hkv + g) * Kt;
        for (int k = 0; k < Kt; ++k) dw[so + k] = 0.0;
        for (int k = 0; k < Kt; ++k) ds[so + k] = 0.0;
        /* With masks, a row is needed if its dQ is asked for or it selected a chunk whose
         * gradients are asked for (phase 2 reads that row's ds). */
        int need = want_q || !chunk_mask;
        for (int k = 0; k < Kt && !need; ++k)
          if (idx[so + k] >= 0 && chunk_mask[(size_t)b * nC + idx[so + k]]) need = 1;
        if (!need) continue;
        if (want_q)
          for (int hh = 0; hh < G; ++hh) {
            double* dq = dQ + (((size_t)b * L + t) * Hq + g * G + hh) * D;
            for (int e = 0; e < D; ++e) dq[e] = 0.0;
          }
        for (int k = 0; k < Kt; ++k) {
          int c = idx[so + k];
          if (c < 0) continue;
          size_t k0 = (((size_t)b * L + (size_t)c * S) * Hkv + g) * D;
          for (int h = 0; h < Hq; ++h) {
            if (group_of(h, Hq, Hkv) != g) continue;
            size_t qoff = (((size_t)b * L + t) * Hq + h) * D;
            softmax1_probs(Q, dt, qoff, K, dt, k0, kstride, D, S, sm_scale, a);
            double Dhk = 0.0;
            for (int j = 0; j < S; ++j) {
              double s = 0.0;
              for (int e = 0; e < D; ++e) s += ld(dO, qoff + e, dt) * ld(V, k0 + j * kstride + e, dt);
              dA[j] = s;
              Dhk += a[j] * s;
            }
            dw[so + k] += Dhk;
            if (!want_q) continue;
            double* dq = dQ + qoff;
            for (int j = 0; j < S; ++j) {
              double dz = w[so + k] * a[j] * (dA[j] - Dhk);
              for (int e = 0; e < D; ++e) dq[e] += sm_scale * dz * ld(K, k0 + j * kstride + e, dt);
            }
          }
        }
        if (wmode == ORC_W_SOFTMAX) {
          /* softmax backward over the valid slots */
          double mean = 0.0; /* sum_j w_j dw_j */
          for (int k = 0; k < Kt; ++k)
            if (idx[so + k] >= 0) mean += w[so + k] * dw[so + k];
          for (int k = 0; k < Kt; ++k)
            ds[so + k] = idx[so + k] < 0 ? 0.0
                                         : w[so + k] * (dw[so + k] - (MUT(11) ? 0.0 : mean));
        } else {
          /* stick-breaking backward over the valid slots (they are a prefix) */
          double suffix = 0.0; /* sum_{k'>k} dw_k' w_k' */
          for (int k = Kt - 1; k >= 0; --k) {
            if (idx[so + k] < 0) {
              ds[so + k] = 0.0;
              continue;
            }
            double p = sigmoid(score[so + k]);
            ds[so + k] = dw[so + k] * w[so + k] * (1.0 - p) - (MUT(6) ? 0.0 : p * suffix);
            suffix += dw[so + k] * w[so + k];
          }
        }
        if (want_q) {
          double* dqs = dQs + (((size_t)b * L + t) * Hkv + g) * D;
          for (int e = 0; e < D; ++e) dqs[e] = 0.0;
          for (int k = 0; k < Kt; ++k) {
            int c = idx[so + k];
            if (c < 0) continue;
            const double* krow = Kslc + (((size_t)b * nC + c) * Hkv + g) * D;
            size_t qso = (((size_t)b * L + t) * Hkv + g) * D;
            for (int e = 0; e < D; ++e)
              dqs[e] += sel_scale * ds[so + k] * (MUT(8) ? ld(Qs, qso + e, dt) : krow[e]);
          }
        }
      }
    }

  /* Phase 2: per chunk, over every (token, slot) that selected it, in token order. */
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g)
      for (int c = 0; c < nC; ++c) {
        if (chunk_mask && !chunk_mask[(size_t)b * nC + c]) continue;
        double a[1024], dA[1024];
        size_t k0 = (((size_t)b * L + (size_t)c * S) * Hkv + g) * D;
        double* dks = dKslc + (((size_t)b * nC + c) * Hkv + g) * D;
        for (int e = 0; e < D; ++e) dks[e] = 0.0;
        for (int j = 0; j < S; ++j)
          for (int e = 0; e < D; ++e) {
            dK[k0 + j * kstride + e] = 0.0;
            dV[k0 + j * kstride + e] = 0.0;
          }
        for (int t = 0; t < L; ++t)
          for (int k = 0; k < Kt; ++k) {
            size_t so = (((size_t)b * L + t) * Hkv + g) * Kt + k;
            if (idx[so] != c) continue;
            for (int h = 0; h < Hq; ++h) {
              if (group_of(h, Hq, Hkv) != g) continue;
              size_t qoff = (((size_t)b * L + t) * Hq + h) * D;
              softmax1_probs(Q, dt, qoff, K, dt, k0, kstride, D, S, sm_scale, a);
              double Dhk = 0.0;
              for (int j = 0; j < S; ++j) {
                double s = 0.0;
                for (int e = 0; e < D; ++e) s += ld(dO, qoff + e, dt) * ld(V, k0 + j * kstride + e, dt);
                dA[j] = s;
                Dhk += a[j] * s;
              }
              for (int j = 0; j < S; ++j) {
                double wa = (MUT(7) ? 1.0 : w[so]) * a[j];
                double dz = w[so] * a[j] * (dA[j] - Dhk);
                for (int e = 0; e < D; ++e) {
                  dV[k0 + j * kstride + e] += wa * ld(dO, qoff + e, dt);
                  dK[k0 + j * kstride + e] += sm_scale * dz * ld(Q, qoff + e, dt);
                }
              }
            }
            size_t qso = (((size_t)b * L + t) * Hkv + g) * D;
            for (int e = 0; e < D; ++e) dks[e] += sel_scale * ds[so] * ld(Qs, qso + e, dt);
          }
        if (fold)
          for (int j = 0; j < S; ++j)
            for (int e = 0; e < D; ++e) dK[k0 + j * kstride + e] += dks[e] / S;
      }

  /* Key/value rows of the incomplete tail chunk are never selected. */
  for (int b = 0; b < B; ++b)
    for (int t = nC * S; t < L; ++t)
      for (int g = 0; g < Hkv; ++g)
        for (int e = 0; e < D; ++e) {
          dK[(((size_t)b * L + t) * Hkv + g) * D + e] = 0.0;
          dV[(((size_t)b * L + t) * Hkv + g) * D + e] = 0.0;
        }
}

/* ---- Decode: one new query per sequence against the resident chunk table ------------
 * [HSA-note 训练与推理优化, "KV Cache Offloading"]: at inference only the compact chunk
 * table stays resident for selection and each step reads only the selected chunks' KV.
 * The new token sits at position ctx, so it may select chunks c < floor(ctx/S).
 * q: [B, Hq, D]; qs: [B, Hkv, D]; Kc, Vc: [B, ctx, Hkv, D]; Kslc: [B, ctx/S, Hkv, D] double.
 * Out: O [B, Hq, D], idx/score/w [B, Hkv, Kt]. */
void oracle_decode(const void* q, const void* qs, const void* Kc, const void* Vc, int dt,
                   const double* Kslc, int B, int ctx, int Hq, int Hkv, int D, int S, int Kt,
                   double sm_scale, double sel_scale, int score_dt, int wmode, double* O,
                   int32_t* idx, double* score, double* w) {
  int nC = ctx / S;
  int n_avail = n_available(ctx, S, nC);
  size_t kstride = (size_t)Hkv * D;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int b = 0; b < B; ++b)
    for (int g = 0; g < Hkv; ++g) {
      cand_t* cand = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n_avail > 0 ? n_avail : 1));
      size_t qso = ((size_t)b * Hkv + g) * D;
      for (int c = 0; c < n_avail; ++c) {
        const double* krow = Kslc + (((size_t)b * nC + c) * Hkv + g) * D;
        cand[c].s = sel_score(qs, dt, qso, krow, D, sel_scale, score_dt);
        cand[c].c = c;
      }
      size_t so = ((size_t)b * Hkv + g) * Kt;
      select_row(cand, n_avail, Kt, wmode, idx + so, score + so, w + so);
      free(cand);
      double a[1024];
      for (int h = 0; h < Hq; ++h) {
        if (group_of(h, Hq, Hkv) != g) continue;
        size_t qoff = ((size_t)b * Hq + h) * D;
        double* out = O + qoff;
        for (int e = 0; e < D; ++e) out[e] = 0.0;
        for (int k = 0; k < Kt; ++k) {
          int c = idx[so + k];
          if (c < 0) continue;
          size_t k0 = (((size_t)b * ctx + (size_t)c * S) * Hkv + g) * D;
          softmax1_probs(q, dt, qoff, Kc, dt, k0, kstride, D, S, sm_scale, a);
          for (int e = 0; e < D; ++e) {
            double acc = 0.0;
            for (int j = 0; j < S; ++j) acc += a[j] * ld(Vc, k0 + j * kstride + e, dt);
            out[e] += w[so + k] * acc;
          }
        }
      }
    }
}
