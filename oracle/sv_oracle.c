/*
 * sv_oracle.c -- CPU oracle (double precision) for batched verification of
 * draft blocks against target logits.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline; never by the GPU library.  It shares no code with
 * the GPU path.  Every function follows the definition written in its
 * comment, in plain loops, without blocking, fusion or reordering; a library
 * sort (qsort) and libm exp/log are the only primitives.
 *
 * Sources are listed in sv_oracle.h ([DScale], [DBLast], [wispaper], [Philox]).
 */
#include "sv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 [Philox]: ten rounds of a 2x(32x32->64) multiply round.   */
/* Per round, with multipliers M0, M1 and the current key (k0, k1):          */
/*   (hi0, lo0) = M0 * c0,  (hi1, lo1) = M1 * c2                             */
/*   c' = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)                           */
/* and the key advances by the Weyl constants (W0, W1) between rounds.       */
/* ------------------------------------------------------------------------ */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * (uint64_t)c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
  memcpy(out, c, sizeof c);
}

/* 24 high bits of a word as a uniform on the grid {0, 2^-24, ..., 1 - 2^-24} */
double orc_u24(uint32_t w) { return (double)(w >> 8) * (1.0 / 16777216.0); }

/* The uniforms of request r at 0-based position i come from the counter
 * (i, r, 0, 0) under key = (low 32 bits of seed, high 32 bits of seed). */
static void orc_words_at(uint64_t seed, int32_t r, int32_t i, uint32_t w[4]) {
  uint32_t ctr[4] = {(uint32_t)i, (uint32_t)r, 0u, 0u};
  uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  orc_philox4x32_10(ctr, key, w);
}

void orc_uniform_words(uint64_t seed, int32_t R, int32_t n_pos, uint32_t* out) {
  for (int32_t r = 0; r < R; ++r)
    for (int32_t i = 0; i < n_pos; ++i) orc_words_at(seed, r, i, out + ((size_t)r * n_pos + i) * 4);
}

/* ------------------------------------------------------------------------ */
/* logit values                                                              */
/* ------------------------------------------------------------------------ */
static double orc_val(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == ORC_F32) return (double)((const float*)base)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static const void* orc_row(const void* base, int32_t dtype, int64_t row, int64_t ld) {
  size_t es = dtype == ORC_F32 ? 4 : 2;
  return (const char*)base + (size_t)row * (size_t)ld * es;
}

/* ------------------------------------------------------------------------ */
/* DVL allocation [DScale abstract: a verification budget of half the       */
/* full-length capacity goes to the best-scored draft prefixes; wispaper:    */
/* prefixes are scored by how likely they are to survive verification].      */
/* Reading: the score of a prefix of length i is its survival probability    */
/* s_i = a_1 * ... * a_i (products rounded to float one at a time); the      */
/* allocation maximises the summed score of the verified positions under the  */
/* budget.  Since every a <= 1 the scores fall along a request, so the        */
/* budget best positions in the order (s desc, r asc, i asc) are prefix-closed */
/* and form the optimum.                                                     */
/* ------------------------------------------------------------------------ */
typedef struct {
  float s;
  int32_t r, i;
} orc_dvl_item;

static int orc_dvl_cmp(const void* pa, const void* pb) {
  const orc_dvl_item* x = (const orc_dvl_item*)pa;
  const orc_dvl_item* y = (const orc_dvl_item*)pb;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  if (x->r != y->r) return x->r < y->r ? -1 : 1;
  if (x->i != y->i) return x->i < y->i ? -1 : 1;
  return 0;
}

/* Per-request block length [wispaper Q&A on block-diffusion decode failures, */
/* section "Why is a fixed block size a failure mode in production?":         */
/* BlockPilot finds the best block size varies from request to request]:     */
/* request r drafts b_r <= b                                                  */
/* positions; positions i >= b_r were not drafted, are never candidates and   */
/* get score 0.  block_len NULL: b_r = b.  Returns 2 if some b_r lies outside */
/* [0, b] (nothing written).                                                  */
int orc_dvl_ragged(const float* a, int32_t R, int32_t b, const int32_t* block_len, int32_t budget, float* s,
                   int32_t* L, int32_t* pos_off, int32_t* tgt_off) {
  int bad = 0;
  if (block_len)
    for (int32_t r = 0; r < R; ++r)
      if (block_len[r] < 0 || block_len[r] > b) return 2;
  size_t n = 0; /* candidates */
  for (int32_t r = 0; r < R; ++r) {
    const int32_t br = block_len ? block_len[r] : b;
    float run = 1.0f;
    for (int32_t i = 0; i < b; ++i) {
      if (i >= br) {
        s[(size_t)r * b + i] = 0.0f;
        continue;
      }
      const float av = a[(size_t)r * b + i];
      if (!(av >= 0.0f && av <= 1.0f)) bad = 1;
      float prod = run * av; /* one float rounding per step */
      s[(size_t)r * b + i] = prod;
      run = prod;
    }
    n += (size_t)br;
  }
  orc_dvl_item* items = (orc_dvl_item*)malloc(sizeof(orc_dvl_item) * (n ? n : 1));
  size_t k0 = 0;
  for (int32_t r = 0; r < R; ++r) {
    const int32_t br = block_len ? block_len[r] : b;
    for (int32_t i = 0; i < br; ++i) {
      items[k0].s = s[(size_t)r * b + i];
      items[k0].r = r;
      items[k0].i = i;
      ++k0;
    }
  }
  qsort(items, n, sizeof(orc_dvl_item), orc_dvl_cmp);
  size_t take = budget <= 0 ? 0 : ((size_t)budget < n ? (size_t)budget : n);
  for (int32_t r = 0; r < R; ++r) L[r] = 0;
  for (size_t k = 0; k < take; ++k) L[items[k].r] += 1;
  free(items);
  pos_off[0] = 0;
  tgt_off[0] = 0;
  for (int32_t r = 0; r < R; ++r) {
    pos_off[r + 1] = pos_off[r] + L[r];
    tgt_off[r + 1] = tgt_off[r] + L[r] + 1;
  }
  return bad;
}

int orc_dvl(const float* a, int32_t R, int32_t b, int32_t budget, float* s, int32_t* L,
            int32_t* pos_off, int32_t* tgt_off) {
  return orc_dvl_ragged(a, R, b, NULL, budget, s, L, pos_off, tgt_off);
}

double orc_dvl_objective(const float* s, const int32_t* L, int32_t R, int32_t b) {
  double acc = 0.0;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t i = 0; i < L[r]; ++i) acc += (double)s[(size_t)r * b + i];
  return acc;
}

/* ------------------------------------------------------------------------ */
/* Target sampling filter [DBLast review, "What would settle it": sampling   */
/* at temperature T with top-p; reference graph [18], nucleus sampling].     */
/*   p = softmax(l / T); with top-p: order the tokens by (l desc, index asc), */
/*   accumulate p, and stop at the first token where the running sum reaches */
/*   top_p; its logit is the cut; keep every token with l >= cut (ties kept) */
/*   and renormalise.  T = 0 means greedy: p is one-hot at the argmax.       */
/* ------------------------------------------------------------------------ */
typedef struct {
  double v;
  int32_t idx;
} orc_sort_item;

static int orc_desc_cmp(const void* pa, const void* pb) {
  const orc_sort_item* x = (const orc_sort_item*)pa;
  const orc_sort_item* y = (const orc_sort_item*)pb;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);
}

void orc_row_stats(const void* row, int32_t dtype, int32_t V, double T, double top_p,
                   orc_row_stats_t* out) {
  double m = -INFINITY;
  int32_t am = 0;
  for (int32_t v = 0; v < V; ++v) {
    double l = orc_val(row, dtype, v);
    if (l > m) { /* strict: the lowest index wins ties */
      m = l;
      am = v;
    }
  }
  out->max = (float)m;
  out->argmax = am;
  out->margin = INFINITY;
  if (T == 0.0) {
    out->lse = 0.0;
    out->cut = (float)m;
    out->kept_lse = 0.0;
    return;
  }
  /* lse = log sum_v exp(l_v / T), evaluated as M + log sum exp(l_v/T - M) */
  double M = m / T;
  double S = 0.0;
  for (int32_t v = 0; v < V; ++v) S += exp(orc_val(row, dtype, v) / T - M);
  double lse = M + log(S);
  out->lse = lse;
  if (!(top_p < 1.0)) {
    out->cut = -INFINITY;
    out->kept_lse = lse;
    return;
  }
  orc_sort_item* it = (orc_sort_item*)malloc(sizeof(orc_sort_item) * (size_t)V);
  for (int32_t v = 0; v < V; ++v) {
    it[v].v = orc_val(row, dtype, v);
    it[v].idx = v;
  }
  qsort(it, (size_t)V, sizeof(orc_sort_item), orc_desc_cmp);
  double cut = it[V - 1].v; /* if rounding keeps the sum below top_p: keep all */
  double run = 0.0;
  for (int32_t k = 0; k < V; ++k) {
    run += exp(it[k].v / T - lse);
    if (run >= top_p) {
      cut = it[k].v;
      break;
    }
  }
  free(it);
  double c_gt = 0.0, c_ge = 0.0, kept = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    double l = orc_val(row, dtype, v);
    double p = exp(l / T - lse);
    if (l > cut) c_gt += p;
    if (l >= cut) {
      c_ge += p;
      kept += exp(l / T - M);
    }
  }
  out->cut = (float)cut;
  out->kept_lse = M + log(kept);
  out->margin = fmin(fabs(c_gt - top_p), fabs(c_ge - top_p));
}

void orc_row_stats_batch(const void* rows, int32_t dtype, int64_t ld, int32_t V, int32_t nrows,
                         const int32_t* req, const float* T, const float* top_p,
                         orc_row_stats_t* out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int32_t k = 0; k < nrows; ++k) {
    int32_t r = req[k];
    double tp = top_p ? (double)top_p[r] : 1.0;
    orc_row_stats(orc_row(rows, dtype, k, ld), dtype, V, (double)T[r], tp, &out[k]);
  }
}

static int32_t orc_argmax_row(const void* row, int32_t dtype, int32_t V) {
  double m = -INFINITY;
  int32_t am = 0;
  for (int32_t v = 0; v < V; ++v) {
    double l = orc_val(row, dtype, v);
    if (l > m) {
      m = l;
      am = v;
    }
  }
  return am;
}

void orc_argmax_rows(const void* rows, int32_t dtype, int64_t ld, int32_t V, int32_t nrows,
                     int32_t* out) {
#pragma omp parallel for schedule(dynamic, 4)
  for (int32_t k = 0; k < nrows; ++k) out[k] = orc_argmax_row(orc_row(rows, dtype, k, ld), dtype, V);
}

/* target probability of token v under row statistics st (T > 0 or T == 0) */
static double orc_p_of(const void* row, int32_t dtype, int32_t v, double T,
                       const orc_row_stats_t* st) {
  if (T == 0.0) return v == st->argmax ? 1.0 : 0.0;
  double l = orc_val(row, dtype, v);
  if (l < (double)st->cut) return 0.0;
  return exp(l / T - st->kept_lse);
}

/* ------------------------------------------------------------------------ */
/* Draft conditionals.                                                       */
/* Dense (independent block drafter): q_i = softmax(d_i / T), one-hot argmax */
/* at T = 0, no top-p.                                                       */
/* Mixture [DBLast review, "What carries the argument"]:                     */
/*   q_dep(x_1:b | y) = sum_z q(z|y) prod_i q_i(x_i | y, z),  q(z|y) =       */
/*   softmax(mixing logits).  The conditional of position i given the draft  */
/*   prefix x_<i is  q(v | x_<i) = sum_z w_z^(i) q_i(v | z)  with the        */
/*   category posterior  w_z^(i) proportional to q(z|y) prod_{j<i} q_j(x_j|z) */
/*   (Bayes' rule on the mixture).  Greedy branches (Eq. (18)/(20) of the     */
/*   paper as the review cites them): q_i(. | z) is a point mass at the      */
/*   branch's argmax g_i(z); soft branches: softmax(c / branch_T).           */
/*   If no branch is consistent with the prefix the posterior is empty and   */
/*   q is zero everywhere.                                                    */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t K, b, V, dtype;
  double branch_T;
  const void* comp;
  int64_t ld, row0;
  int32_t* g;       /* [K*b] greedy branch tokens */
  double* lse;      /* [K*b] soft branch lse (branch_T > 0) */
  double* logpost;  /* [K] running log q(z|y) + sum_j log q_j(x_j|z) */
} orc_mix_t;

static const void* orc_comp_row(const orc_mix_t* mx, int32_t z, int32_t i) {
  return orc_row(mx->comp, mx->dtype, mx->row0 + (int64_t)z * mx->b + i, mx->ld);
}

/* log q_i(v | z) */
static double orc_branch_logq(const orc_mix_t* mx, int32_t z, int32_t i, int32_t v) {
  if (mx->branch_T == 0.0) return mx->g[z * mx->b + i] == v ? 0.0 : -INFINITY;
  return orc_val(orc_comp_row(mx, z, i), mx->dtype, v) / mx->branch_T - mx->lse[z * mx->b + i];
}

/* normalised posterior weights w (K) from the running log weights */
static void orc_posterior(const orc_mix_t* mx, double* w) {
  double mx_l = -INFINITY;
  for (int32_t z = 0; z < mx->K; ++z) mx_l = fmax(mx_l, mx->logpost[z]);
  if (mx_l == -INFINITY) {
    for (int32_t z = 0; z < mx->K; ++z) w[z] = 0.0;
    return;
  }
  double tot = 0.0;
  for (int32_t z = 0; z < mx->K; ++z) {
    w[z] = exp(mx->logpost[z] - mx_l);
    tot += w[z];
  }
  for (int32_t z = 0; z < mx->K; ++z) w[z] /= tot;
}

/* q(v | x_<i) given posterior weights w before position i */
static double orc_mix_q(const orc_mix_t* mx, const double* w, int32_t i, int32_t v) {
  double q = 0.0;
  for (int32_t z = 0; z < mx->K; ++z) {
    if (w[z] == 0.0) continue;
    double lq = orc_branch_logq(mx, z, i, v);
    if (lq != -INFINITY) q += w[z] * exp(lq);
  }
  return q;
}

/* ------------------------------------------------------------------------ */
/* Inverse-CDF draw over the vocabulary in index order: the smallest v whose */
/* running sum C_v exceeds u * W.  If rounding leaves no such v the largest  */
/* v with positive weight is taken.  Margin: distance of u*W to the ends of  */
/* the chosen interval, divided by W.                                        */
/* ------------------------------------------------------------------------ */
static int32_t orc_inverse_cdf(const double* w, int32_t V, double u, double* margin) {
  double W = 0.0;
  for (int32_t v = 0; v < V; ++v) W += w[v];
  double t = u * W;
  double run = 0.0;
  for (int32_t v = 0; v < V; ++v) {
    double prev = run;
    run += w[v];
    if (run > t) {
      *margin = fmin(t - prev, run - t) / W;
      return v;
    }
  }
  for (int32_t v = V - 1; v >= 0; --v)
    if (w[v] > 0.0) {
      *margin = 0.0;
      return v;
    }
  *margin = 0.0;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* One verification step [DBLast review, "Assumptions": speculative sampling */
/* with rejection correction (reference graph [1], [2])], per request r:     */
/*   for i = 1..L_r: accept x_i iff u_acc < p_i(x_i) / q_i(x_i | x_<i)        */
/*     (q = 0: accept iff p > 0); the first rejection ends the block;        */
/*   on a rejection at position j: sample from norm(max(0, p_j - q_j))        */
/*     (all-zero residual from rounding: sample from p_j);                    */
/*   if all L_r are accepted: a bonus sample from p_{L_r + 1}.               */
/* u_acc is word 0 and the sample's uniform word 1 of Philox at counter      */
/* (i - 1, r, 0, 0), i the 1-based position of the decision.                 */
/* ------------------------------------------------------------------------ */
int orc_step(const orc_step_in_t* in, const orc_step_out_t* out) {
  const int32_t R = in->R, b = in->b, V = in->V, K = in->K;
  if (R < 0 || b < 1 || V < 1) return 1;
  if (in->q_mode == ORC_Q_MIXTURE && K < 1) return 1;
  for (int32_t r = 0; r < R; ++r)
    if (in->L[r] < 0 || in->L[r] > b) return 2;
  int err = 0;
#pragma omp parallel
  {
    double* wbuf = (double*)malloc(sizeof(double) * (size_t)V);
    orc_row_stats_t* st = (orc_row_stats_t*)malloc(sizeof(orc_row_stats_t) * (size_t)(b + 1));
    orc_row_stats_t* dst = (orc_row_stats_t*)malloc(sizeof(orc_row_stats_t) * (size_t)b);
    int32_t* g = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1) * b);
    double* blse = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * b);
    double* logpost = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double* wpost = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * (b + 1));
#pragma omp for schedule(dynamic, 1)
    for (int32_t r = 0; r < R; ++r) {
      const int32_t Lr = in->L[r];
      const double T = (double)in->T[r];
      const double tp = in->top_p ? (double)in->top_p[r] : 1.0;
      const int32_t* x = in->x + (size_t)r * b;
      int bad_tok = 0;
      for (int32_t i = 0; i < Lr; ++i)
        if (x[i] < 0 || x[i] >= V) bad_tok = 1;
      if (bad_tok) {
#pragma omp atomic write
        err = 3;
        continue;
      }
      /* target rows 0..Lr */
      for (int32_t j = 0; j <= Lr; ++j)
        orc_row_stats(orc_row(in->tgt, in->dtype, in->tgt_row0[r] + j, in->tgt_ld), in->dtype, V, T,
                      tp, &st[j]);
      /* draft conditionals at the draft tokens */
      orc_mix_t mx;
      memset(&mx, 0, sizeof mx);
      if (in->q_mode == ORC_Q_DENSE) {
        for (int32_t i = 0; i < Lr; ++i)
          orc_row_stats(orc_row(in->draft, in->dtype, in->draft_row0[r] + i, in->draft_ld), in->dtype,
                        V, T, 1.0, &dst[i]);
      } else {
        mx.K = K;
        mx.b = b;
        mx.V = V;
        mx.dtype = in->dtype;
        mx.branch_T = in->branch_T;
        mx.comp = in->comp;
        mx.ld = in->comp_ld;
        mx.row0 = in->comp_row0[r];
        mx.g = g;
        mx.lse = blse;
        mx.logpost = logpost;
        for (int32_t z = 0; z < K; ++z)
          for (int32_t i = 0; i < Lr; ++i) {
            const void* row = orc_comp_row(&mx, z, i);
            if (in->branch_T == 0.0) {
              g[z * b + i] = orc_argmax_row(row, in->dtype, V);
            } else {
              orc_row_stats_t bs;
              orc_row_stats(row, in->dtype, V, in->branch_T, 1.0, &bs);
              blse[z * b + i] = bs.lse;
              g[z * b + i] = bs.argmax;
            }
          }
        /* q(z | y) = softmax(mixing logits) */
        const float* ml = in->mix + (size_t)r * K;
        double mmax = -INFINITY, msum = 0.0;
        for (int32_t z = 0; z < K; ++z) mmax = fmax(mmax, (double)ml[z]);
        for (int32_t z = 0; z < K; ++z) msum += exp((double)ml[z] - mmax);
        for (int32_t z = 0; z < K; ++z) logpost[z] = ((double)ml[z] - mmax) - log(msum);
        /* posterior before each position, conditioned on the draft prefix */
        for (int32_t i = 0; i <= Lr && i < b; ++i) {
          orc_posterior(&mx, wpost + (size_t)i * K);
          if (i < Lr)
            for (int32_t z = 0; z < K; ++z) logpost[z] += orc_branch_logq(&mx, z, i, x[i]);
        }
        if (out->branch_tok)
          for (int32_t z = 0; z < K; ++z)
            for (int32_t i = 0; i < Lr; ++i) out->branch_tok[((size_t)r * K + z) * b + i] = g[z * b + i];
        if (out->post_w)
          for (int32_t i = 0; i < Lr; ++i)
            for (int32_t z = 0; z < K; ++z)
              out->post_w[((size_t)r * b + i) * K + z] = wpost[(size_t)i * K + z];
      }
      /* acceptance tests */
      int32_t n_acc = Lr;
      for (int32_t i = 0; i < Lr; ++i) {
        const void* trow = orc_row(in->tgt, in->dtype, in->tgt_row0[r] + i, in->tgt_ld);
        double p = orc_p_of(trow, in->dtype, x[i], T, &st[i]);
        double q;
        if (in->q_mode == ORC_Q_DENSE) {
          const void* drow = orc_row(in->draft, in->dtype, in->draft_row0[r] + i, in->draft_ld);
          if (T == 0.0)
            q = x[i] == dst[i].argmax ? 1.0 : 0.0;
          else
            q = exp(orc_val(drow, in->dtype, x[i]) / T - dst[i].lse);
        } else {
          q = orc_mix_q(&mx, wpost + (size_t)i * K, i, x[i]);
        }
        uint32_t w[4];
        orc_words_at(in->seed, r, i, w);
        double u = orc_u24(w[0]);
        int accept;
        double margin;
        if (q > 0.0) {
          double rho = p / q;
          accept = u < rho;
          margin = fabs(u - fmin(1.0, rho));
        } else {
          accept = p > 0.0;
          margin = accept ? 1.0 - u : u;
        }
        size_t k = (size_t)r * b + i;
        if (out->u_acc) out->u_acc[k] = u;
        if (out->p_x) out->p_x[k] = p;
        if (out->q_x) out->q_x[k] = q;
        if (out->acc_margin) out->acc_margin[k] = margin;
        if (!accept && n_acc == Lr) n_acc = i;
      }
      /* residual (n_acc < Lr) or bonus (n_acc == Lr) sample from row n_acc */
      const int32_t j = n_acc;
      const int bonus = n_acc == Lr;
      const void* trow = orc_row(in->tgt, in->dtype, in->tgt_row0[r] + j, in->tgt_ld);
      uint32_t w4[4];
      orc_words_at(in->seed, r, j, w4);
      double u1 = orc_u24(w4[1]);
      double W = 0.0;
      for (int32_t v = 0; v < V; ++v) {
        double p = orc_p_of(trow, in->dtype, v, T, &st[j]);
        double q = 0.0;
        if (!bonus) {
          if (in->q_mode == ORC_Q_DENSE) {
            const void* drow = orc_row(in->draft, in->dtype, in->draft_row0[r] + j, in->draft_ld);
            q = T == 0.0 ? (v == dst[j].argmax ? 1.0 : 0.0)
                         : exp(orc_val(drow, in->dtype, v) / T - dst[j].lse);
          } else {
            q = orc_mix_q(&mx, wpost + (size_t)j * K, j, v);
          }
        }
        wbuf[v] = p - q > 0.0 ? p - q : 0.0;
        W += wbuf[v];
      }
      if (!(W > 0.0)) /* p == q up to rounding: fall back to p */
        for (int32_t v = 0; v < V; ++v) wbuf[v] = orc_p_of(trow, in->dtype, v, T, &st[j]);
      double sm;
      int32_t tok = orc_inverse_cdf(wbuf, V, u1, &sm);
      out->n_acc[r] = n_acc;
      out->token[r] = tok;
      out->is_bonus[r] = bonus;
      if (out->sample_margin) out->sample_margin[r] = sm;
      if (out->u_res) out->u_res[r] = u1;
    }
    free(wbuf);
    free(st);
    free(dst);
    free(g);
    free(blse);
    free(logpost);
    free(wpost);
  }
  return err;
}


/* ------------------------------------------------------------------------ */
/* Tree verification.  The pages name tree drafters (wispaper Q&A on         */
/* block-diffusion decode failures, section "Why is a fixed block size a      */
/* failure mode in production?": Bastion's budget-aware draft trees; its      */
/* source list: D2SD's confidence-guided prefix trees) but give no rule for   */
/* verifying several candidates.  Reading: multi-round speculative sampling   */
/* (Miao et al., SpecInfer, ASPLOS 2024) -- the candidates at a node were     */
/* drawn independently from the drafter's distribution q of that position,    */
/* and are tested in turn:                                                    */
/*   start at the root with the current target r = p (the node's target);   */
/*   child j with token x: accept iff u_j < r(x) / q(x) (q = 0: iff r(x) > 0); */
/*   on acceptance move to j and start again with p of node j;                */
/*   on rejection replace r by norm(max(0, r - q)) and try the next child;    */
/*   when every child is rejected, draw the token from that residual;         */
/*   at a node without children, draw a bonus token from its p.              */
/* Each round is one speculative-sampling step between r and q, so the        */
/* emitted token follows p whatever q is ("Pith review of DBLAST",            */
/* "Assumptions & free parameters": rejection correction keeps the target).  */
/* Uniforms: the test of node j takes word 0 at counter (j - 1, r, 0, 0), the */
/* draw at the stopping node s word 1 at (s, r, 0, 0) -- for a chain          */
/* (p(j) = j - 1) the counters and arithmetic of orc_step.  A residual that   */
/* rounding leaves empty is replaced by p (as in orc_step).                  */
/* ------------------------------------------------------------------------ */
int orc_tree_step(const orc_tree_in_t* in, const orc_tree_out_t* out) {
  const int32_t R = in->R, b = in->b, V = in->V;
  if (R < 0 || b < 1 || V < 1 || !in->node_off || in->node_off[0] != 0) return 1;
  for (int32_t r = 0; r < R; ++r) {
    const int32_t n0 = in->node_off[r], N = in->node_off[r + 1] - n0;
    if (N < 1 || in->parent[n0] != -1) return 2;
    for (int32_t j = 1; j < N; ++j) {
      const int32_t pj = in->parent[n0 + j], tj = in->token[n0 + j];
      if (pj < 0 || pj >= j || tj < 0 || tj >= V) return 2;
    }
  }
  int err = 0;
#pragma omp parallel
  {
    double* pcur = (double*)malloc(sizeof(double) * (size_t)V);
    double* wbuf = (double*)malloc(sizeof(double) * (size_t)V);
#pragma omp for schedule(dynamic, 1)
    for (int32_t r = 0; r < R; ++r) {
      const int32_t n0 = in->node_off[r], N = in->node_off[r + 1] - n0;
      const int32_t* par = in->parent + n0;
      const int32_t* tok = in->token + n0;
      const double T = (double)in->T[r];
      const double tp = in->top_p ? (double)in->top_p[r] : 1.0;
      int32_t* depth = (int32_t*)malloc(sizeof(int32_t) * (size_t)N);
      depth[0] = 0;
      int bad = 0;
      for (int32_t j = 1; j < N; ++j) {
        depth[j] = depth[par[j]] + 1;
        if (depth[j] > b) bad = 1;
      }
      if (bad) {
        free(depth);
#pragma omp atomic write
        err = 3;
        continue;
      }
      int32_t u = 0, n = 0;
      for (;;) {
        const void* trow = orc_row(in->tgt, in->dtype, in->tgt_row[n0 + u], in->tgt_ld);
        orc_row_stats_t st;
        orc_row_stats(trow, in->dtype, V, T, tp, &st);
        int32_t first = -1;
        for (int32_t j = u + 1; j < N; ++j)
          if (par[j] == u) {
            first = j;
            break;
          }
        uint32_t w4[4];
        if (first < 0) { /* a leaf: bonus token from p */
          for (int32_t v = 0; v < V; ++v) wbuf[v] = orc_p_of(trow, in->dtype, v, T, &st);
          orc_words_at(in->seed, r, u, w4);
          double sm;
          out->token[r] = orc_inverse_cdf(wbuf, V, orc_u24(w4[1]), &sm);
          out->is_bonus[r] = 1;
          if (out->sample_margin) out->sample_margin[r] = sm;
          if (out->u_res) out->u_res[r] = orc_u24(w4[1]);
          break;
        }
        /* the drafter's distribution of this position: draft row depth(u) */
        const void* drow = orc_row(in->draft, in->dtype, in->draft_row0[r] + depth[u], in->draft_ld);
        orc_row_stats_t dst;
        orc_row_stats(drow, in->dtype, V, T, 1.0, &dst);
#define ORC_TREE_Q(v) (T == 0.0 ? ((v) == dst.argmax ? 1.0 : 0.0) : exp(orc_val(drow, in->dtype, (v)) / T - dst.lse))
        int have_res = 0; /* 0: the current target r is p itself */
        double W = 0.0;
        int32_t acc = -1;
        for (int32_t j = first; j < N; ++j) {
          if (par[j] != u) continue;
          const int32_t x = tok[j];
          const double px = have_res ? pcur[x] : orc_p_of(trow, in->dtype, x, T, &st);
          const double qx = ORC_TREE_Q(x);
          orc_words_at(in->seed, r, j - 1, w4);
          const double uu = orc_u24(w4[0]);
          int accept;
          double margin;
          if (qx > 0.0) {
            const double rho = px / qx;
            accept = uu < rho;
            margin = fabs(uu - fmin(1.0, rho));
          } else {
            accept = px > 0.0;
            margin = accept ? 1.0 - uu : uu;
          }
          if (out->u_acc) out->u_acc[n0 + j] = uu;
          if (out->p_x) out->p_x[n0 + j] = px;
          if (out->q_x) out->q_x[n0 + j] = qx;
          if (out->acc_margin) out->acc_margin[n0 + j] = margin;
          if (accept) {
            acc = j;
            break;
          }
          /* rejected: the residual max(0, r - q), normalised for the next child */
          W = 0.0;
          for (int32_t v = 0; v < V; ++v) {
            const double base = have_res ? pcur[v] : orc_p_of(trow, in->dtype, v, T, &st);
            const double d = base - ORC_TREE_Q(v);
            wbuf[v] = d > 0.0 ? d : 0.0;
            W += wbuf[v];
          }
          for (int32_t v = 0; v < V; ++v) pcur[v] = W > 0.0 ? wbuf[v] / W : orc_p_of(trow, in->dtype, v, T, &st);
          have_res = 1;
        }
#undef ORC_TREE_Q
        if (acc >= 0) {
          if (out->path) out->path[(size_t)r * b + n] = acc;
          ++n;
          u = acc;
          continue;
        }
        /* every child rejected: the token from the last residual (from p if rounding emptied it) */
        if (!(W > 0.0))
          for (int32_t v = 0; v < V; ++v) wbuf[v] = orc_p_of(trow, in->dtype, v, T, &st);
        orc_words_at(in->seed, r, u, w4);
        double sm;
        out->token[r] = orc_inverse_cdf(wbuf, V, orc_u24(w4[1]), &sm);
        out->is_bonus[r] = 0;
        if (out->sample_margin) out->sample_margin[r] = sm;
        if (out->u_res) out->u_res[r] = orc_u24(w4[1]);
        break;
      }
      out->n_acc[r] = n;
      out->stop_node[r] = u;
      free(depth);
    }
    free(pcur);
    free(wbuf);
  }
  return err;
}
