/*
 * sv_oracle.h -- CPU oracle for batched speculative-sampling verification.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and sv_oracle.c are the plain, slow,
 * double-precision definition that the GPU library is checked against.  Only
 * the test-suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  The GPU library shares no code, header, table or constant with it.
 *
 * Sources (web pages on the subject; cited by title and section):
 *  [DScale]  "DScale: Scaling Block-Diffusion Speculative Decoding with
 *            Adaptive Verification", abstract (aiqbench.com / arxivdaily.com):
 *            dynamic verify-length (DVL) allocation of a budget of half the
 *            full-length verification capacity to the best-scored prefixes;
 *            buffers at fixed addresses for the per-step lengths.
 *  [DBLast]  "Pith review of DBLAST: Dependent Block Drafting for Stochastic
 *            Speculative Decoding" (pith.science):
 *              - "What carries the argument": latent-mixture proposal
 *                q_dep(x_1:b|y) = sum_z q(z|y) prod_i q_i(x_i|y,z); the
 *                drafter draws one category and emits that branch's argmax
 *                tokens, and the verifier weighs the categories by how well
 *                they explain the draft prefix (the category posterior).
 *              - "Assumptions & free parameters": whatever the proposal q,
 *                the rejection-corrected sampler emits target-distributed
 *                tokens.
 *              - "What would settle it": target sampling at T = 1.5, top-p 0.95.
 *              - Referee report, minor comment 5: experiments use the
 *                conditional of Eq. (20) (greedy-branch proposal).
 *              - Reference graph [1], [2]: Leviathan et al., Chen et al.
 *                (speculative sampling); [18]: nucleus (top-p) sampling.
 *  [wispaper] wispaper.ai Q&A on block-diffusion decode failures, section
 *            "Why does throughput collapse under high concurrency?" (DSpark
 *            sets verification length from how likely each draft prefix is
 *            to survive) and section "Why is a fixed block size a failure
 *            mode in production?" (BlockPilot: block size per request).
 *  [Philox]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *            1, 2, 3", SC'11 -- Philox4x32-10 (outside the pages; the pages
 *            name no generator, the counter-based choice is the build's).
 *
 * Readings where the pages are silent are listed in the repository's design
 * notes; each function below states the one it uses.
 */
#ifndef SV_ORACLE_H
#define SV_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* value types of logit buffers */
#define ORC_F32 0  /* float32 */
#define ORC_BF16 1 /* bfloat16, stored as uint16 bit patterns */

/* ---- Philox4x32-10 [Philox] ------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
/* 24-bit uniform on [0, 1 - 2^-24]: (w >> 8) * 2^-24 */
double orc_u24(uint32_t w);
/* out[(r * n_pos + i) * 4 + k] = word k of Philox(ctr = (i, r, 0, 0), key = seed) */
void orc_uniform_words(uint64_t seed, int32_t R, int32_t n_pos, uint32_t* out);

/* ---- DVL allocation [DScale abstract; wispaper] ------------------------ */
/* s[r*b+i] = fl32(s[r*b+i-1] * a[r*b+i]); choose the min(budget, R*b) best
 * (s desc, r asc, i asc); L[r] = number chosen in r; pos_off / tgt_off are
 * the exclusive scans of L and L+1 (R+1 entries each).  Returns 0, or 1 when
 * an input lies outside [0, 1] (outputs still written). */
int orc_dvl(const float* a, int32_t R, int32_t b, int32_t budget,
            float* s, int32_t* L, int32_t* pos_off, int32_t* tgt_off);
/* The same with a block length b_r per request (block_len[R], NULL = b):
 * only positions i < b_r are candidates; s[r*b+i] = 0 for i >= b_r; the
 * budget is capped at sum_r b_r.  Returns 2 (nothing written) if some b_r
 * lies outside [0, b]; else as orc_dvl (estimates of undrafted positions are
 * not checked). */
int orc_dvl_ragged(const float* a, int32_t R, int32_t b, const int32_t* block_len, int32_t budget,
                   float* s, int32_t* L, int32_t* pos_off, int32_t* tgt_off);
/* objective sum_r sum_{i<L_r} s[r*b+i] in double */
double orc_dvl_objective(const float* s, const int32_t* L, int32_t R, int32_t b);

/* ---- target / draft row statistics ----------------------------------- */
typedef struct {
  float max;        /* largest logit (exact input value) */
  int32_t argmax;   /* lowest index attaining it */
  double lse;       /* log sum_v exp(l_v / T); 0 when T == 0 */
  float cut;        /* top-p cut logit (-inf when top-p is off; max when T == 0) */
  double kept_lse;  /* log sum_{l_v >= cut} exp(l_v / T); lse when off; 0 when T == 0 */
  double margin;    /* top-p decision margin (+inf when off) */
} orc_row_stats_t;

/* statistics of one row of V values; T >= 0, top_p in (0, 1] (>= 1: off) */
void orc_row_stats(const void* row, int32_t dtype, int32_t V, double T, double top_p,
                   orc_row_stats_t* out);
/* nrows rows at rows + k*ld, temperature T[req[k]], top_p[req[k]] (top_p NULL: off) */
void orc_row_stats_batch(const void* rows, int32_t dtype, int64_t ld, int32_t V, int32_t nrows,
                         const int32_t* req, const float* T, const float* top_p,
                         orc_row_stats_t* out);

/* argmax (lowest index on ties) of nrows rows */
void orc_argmax_rows(const void* rows, int32_t dtype, int64_t ld, int32_t V, int32_t nrows,
                     int32_t* out);

/* ---- one verification step ------------------------------------------- */
#define ORC_Q_DENSE 0   /* independent draft: q_i = softmax(d_i / T) */
#define ORC_Q_MIXTURE 1 /* latent mixture of K branches [DBLast] */

typedef struct {
  int32_t R, b, V, K;
  int32_t dtype;            /* ORC_F32 / ORC_BF16 for all logit buffers */
  /* target rows: request r uses rows tgt_row0[r] + j, j = 0..L[r] (L[r]+1 rows) */
  const void* tgt; int64_t tgt_ld; const int64_t* tgt_row0;
  const int32_t* L;         /* verified positions per request, 0 <= L <= b */
  const float* T;           /* [R] temperature (0 = greedy) */
  const float* top_p;       /* [R] or NULL (off) */
  const int32_t* x;         /* [R*b] draft tokens */
  int32_t q_mode;
  /* dense draft: position i (0-based) of r at row draft_row0[r] + i */
  const void* draft; int64_t draft_ld; const int64_t* draft_row0;
  /* mixture: branch z at position i of r at row comp_row0[r] + z*b + i */
  const void* comp; int64_t comp_ld; const int64_t* comp_row0;
  const float* mix;         /* [R*K] mixing logits, q(z|y) = softmax */
  double branch_T;          /* 0: greedy branches; > 0: soft branches softmax(c/branch_T) */
  uint64_t seed;
} orc_step_in_t;

typedef struct {
  int32_t* n_acc;      /* [R] */
  int32_t* token;      /* [R] residual or bonus token */
  int32_t* is_bonus;   /* [R] */
  double* sample_margin; /* [R] */
  double* u_res;       /* [R] uniform used for the sample */
  /* per position (R*b), written for i < L[r]; entries past the first
     rejection are still evaluated (as if that position were reached) */
  double* u_acc;       /* [R*b] */
  double* p_x;         /* [R*b] p_i(x_i) */
  double* q_x;         /* [R*b] q_i(x_i | x_<i) */
  double* acc_margin;  /* [R*b] */
  /* mixture only (may be NULL): branch tokens [R*K*b] (greedy) and
     posterior weights before position i, [R*b*K] */
  int32_t* branch_tok;
  double* post_w;
} orc_step_out_t;

/* Returns 0, or a nonzero code for malformed input. */
int orc_step(const orc_step_in_t* in, const orc_step_out_t* out);

/* ---- tree verification (multi-candidate speculative sampling) -------- */
/* A request's draft is a tree: node 0 is the root (the context so far),
 * node j >= 1 holds a draft token and a parent p(j) < j; the children of a
 * node are tried in increasing index order.  The children of a node at depth
 * d were drawn independently from the drafter's distribution of position
 * d + 1 (a block drafter's position-wise marginal: dense draft row d). */
typedef struct {
  int32_t R, b, V;
  int32_t dtype;             /* ORC_F32 / ORC_BF16 for both logit buffers */
  const int32_t* node_off;   /* [R+1] exclusive scan: request r's nodes are node_off[r] .. node_off[r+1]-1 */
  const int32_t* parent;     /* [node_off[R]] parent of node j (0-based within its request); -1 for the root */
  const int32_t* token;      /* [node_off[R]] draft token of node j (the root's is unused) */
  const void* tgt; int64_t tgt_ld;
  const int64_t* tgt_row;    /* [node_off[R]] target row of node j: p(. | the context and node j's path) */
  const float* T;            /* [R] */
  const float* top_p;        /* [R] or NULL */
  const void* draft; int64_t draft_ld;
  const int64_t* draft_row0; /* [R] children of a node at depth d were drawn from row draft_row0[r] + d */
  uint64_t seed;
} orc_tree_in_t;

typedef struct {
  int32_t* n_acc;        /* [R] accepted nodes */
  int32_t* path;         /* [R*b] the accepted nodes in order (first n_acc[r] entries) */
  int32_t* stop_node;    /* [R] the last accepted node (0: none) */
  int32_t* token;        /* [R] residual or bonus token */
  int32_t* is_bonus;     /* [R] */
  double* sample_margin; /* [R] */
  double* u_res;         /* [R] */
  /* per node ([node_off[R]]), written for the nodes whose test was reached */
  double* u_acc;
  double* p_x;           /* the current target's probability of the node's token */
  double* q_x;           /* the draft's probability of it */
  double* acc_margin;
} orc_tree_out_t;

/* Returns 0, or a nonzero code for malformed input (nothing is written then
 * for the request concerned). */
int orc_tree_step(const orc_tree_in_t* in, const orc_tree_out_t* out);

int orc_num_threads(void);
/* threads for the oracle's later parallel loops (OpenMP); n <= 0 is ignored */
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
