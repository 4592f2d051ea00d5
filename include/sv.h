/*
 * sv.h -- C ABI of libsv: batched verification of block-diffusion draft
 * blocks against target logits on one AMD Instinct MI355X (gfx950).
 *
 * Pages the operations come from (cited by title and section):
 *  [DScale]  "DScale: Scaling Block-Diffusion Speculative Decoding with
 *            Adaptive Verification" -- abstract: dynamic verify-length (DVL)
 *            allocation gives a verification budget of half the full-length
 *            capacity to the best-scored draft prefixes; per-step lengths
 *            reach verification and acceptance through buffers at fixed
 *            addresses.
 *  [DBLast]  "Pith review of DBLAST: Dependent Block Drafting for Stochastic
 *            Speculative Decoding" -- "What carries the argument" (latent
 *            mixture q_dep and the category posterior along the accepted
 *            prefix), "Assumptions & free parameters" (the rejection-
 *            corrected sampler emits tokens distributed as the target),
 *            "What would settle it" (target sampling at temperature 1.5 with
 *            top-p 0.95), Referee report minor 5 (Eq. (20), the greedy-branch
 *            conditional), reference graph [1], [2] (speculative sampling),
 *            [18] (nucleus sampling).
 *  [wispaper] wispaper Q&A on block-diffusion decode failures -- section
 *            "Why does throughput collapse under high concurrency?" (DSpark
 *            sets each request's verification length from the chance that
 *            its draft prefixes survive); section "Why is a fixed block size
 *            a failure mode in production?" (BlockPilot: block size per
 *            request).
 *
 * Conventions shared by every call
 *  - All array arguments are DEVICE pointers unless marked "host".  The caller
 *    owns every buffer; the library allocates nothing and keeps no state
 *    besides the caller's workspace.
 *  - Every per-step value (lengths, offsets, seed, temperature, top-p,
 *    budget) is read from device memory at launch time, so a captured
 *    sequence of calls can be replayed with new values at fixed addresses.
 *    Grids are sized from host-side capacities; work items beyond the
 *    device-side counts exit at once.
 *  - `stream` is a hipStream_t.  Calls are asynchronous; outputs are valid in
 *    stream order.  The workspace holds a status word (updated with atomics,
 *    so calls on different streams may share it), one draw record per
 *    request and the draw's sums per 512-value sub-chunk of the drawn row
 *    (two draws -- sv_residual_sample or sv_accept_sample -- that share a
 *    workspace must not overlap), and sv_verify_rows_dense's split-row part
 *    records and arrival counts (two such calls that share a workspace must
 *    not overlap either).  Only the status word and the arrival counts
 *    (zero between calls, from sv_workspace_init on) outlive a call.
 *  - Requests r = 0..R-1, draft block of b positions, vocabulary V.
 *    L_r = pos_off[r+1] - pos_off[r] is the number of verified positions of
 *    request r (0 <= L_r <= b).  The target gives L_r + 1 rows per request:
 *    rows for positions 1..L_r and the bonus row, packed request after
 *    request at rows tgt_off[r] .. tgt_off[r] + L_r, so tgt_off[r+1] -
 *    tgt_off[r] = L_r + 1.
 *  - Logit rows are row-major with a leading dimension `ld` (elements).  The
 *    base pointer and ld * element size must be multiples of 16 bytes.
 *  - dtype: SV_F32 (float) or SV_BF16 (bfloat16).
 *  - Return value: SV_OK, or an SV_ERR_* code for a host-detectable error, in
 *    which case nothing is launched.  Problems only visible on the device
 *    (bad temperatures, non-finite logits, malformed offsets, ...) set bits
 *    of a sticky status word in the workspace; read it with sv_get_status.
 *    Outputs affected by such a problem are unspecified.
 */
#ifndef SV_H
#define SV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* value types */
#define SV_F32 0
#define SV_BF16 1

/* proposal kinds */
#define SV_Q_DENSE 0   /* independent draft: q_i = softmax(d_i / T_r), one-hot argmax at T_r = 0 */
#define SV_Q_MIXTURE 1 /* latent mixture of K greedy branches [DBLast] */

/* return codes */
#define SV_OK 0
#define SV_ERR_ARG 1       /* null pointer, size out of range, misalignment, unknown dtype/mode */
#define SV_ERR_WORKSPACE 2 /* workspace smaller than sv_workspace_bytes() asks for */
#define SV_ERR_LAUNCH 3    /* the HIP runtime refused a launch or copy */
#define SV_ERR_TOO_LARGE 4 /* problem exceeds SV_NOALLOC_SCRATCH_BYTES (allocation-free entry point) */

/* device status bits (sticky; OR-ed by the kernels) */
#define SV_ST_BAD_TEMPERATURE 0x001u /* T_r < 0 or NaN */
#define SV_ST_BAD_TOP_P 0x002u       /* top_p_r <= 0 or NaN (treated as keeping the top value) */
#define SV_ST_NONFINITE 0x004u       /* NaN or +-Inf in a logit row that was read */
#define SV_ST_BAD_SCORE 0x008u       /* DVL survival estimate outside [0, 1] */
#define SV_ST_BAD_TOKEN 0x010u       /* draft token outside [0, V) */
#define SV_ST_BAD_OFFSETS 0x020u     /* offsets not an exclusive scan, L_r > b, or over capacity */
#define SV_ST_EMPTY_POSTERIOR 0x040u /* no mixture branch consistent with the draft prefix (q = 0) */
#define SV_ST_BAD_BUDGET 0x080u      /* DVL budget < 0 */
#define SV_ST_BAD_NACC 0x100u        /* n_acc outside [0, L_r] */
#define SV_ST_BAD_BLOCK 0x200u       /* DVL block length outside [0, b] (clamped) */
#define SV_ST_BAD_TREE 0x400u        /* a draft tree whose parents, depths, node count or child counts are out of range */

/* ---------------------------------------------------------------- workspace */

/* Bytes of workspace needed for problems of up to R requests, block b,
 * K mixture components (0 if unused) and vocabulary V.  Host-only. */
int32_t sv_workspace_bytes(int32_t R, int32_t b, int32_t K, int32_t V, size_t* out_bytes);

/* Zero the workspace (once, before first use; a fill kernel). */
int32_t sv_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Copy the status word to *host_out, then synchronise the stream. */
int32_t sv_get_status(const void* ws, void* stream, uint32_t* host_out);

/* Reset the status word to 0 (asynchronous, a kernel, no memset). */
int32_t sv_clear_status(void* ws, void* stream);

/* Human-readable text for a return code. */
const char* sv_status_string(int32_t code);

/* ---------------------------------------------------------------- DVL */

/* dvl_alloc_pack [DScale abstract: DVL allocation; wispaper: prefix survival
 * probabilities].
 *   a[R*b]      per-position acceptance estimates in [0, 1] (float)
 *   block_len[R]  optional (NULL: b for every request): request r drafted
 *               only its first b_r positions (0 <= b_r <= b; others clamped,
 *               SV_ST_BAD_BLOCK) [wispaper, section "Why is a fixed block
 *               size a failure mode in production?": BlockPilot's block size
 *               varies per request]; positions i >= b_r are never
 *               chosen and their estimates are ignored (not checked)
 *   budget      device int32 scalar: verification slots B (>= 0)
 *   s[R*b]      out: survival scores s_{r,i} = fl32(s_{r,i-1} * a_{r,i}),
 *               s_{r,0} = a_{r,0}, one float rounding per product; 0 for
 *               i >= b_r
 *   L[R]        out: verified positions per request (L_r <= b_r)
 *   pos_off[R+1], tgt_off[R+1]  out: exclusive scans of L and of L + 1
 * The chosen positions are the min(B, sum_r b_r) best drafted positions in the
 * order (s desc, r asc, i asc); with a <= 1 they are prefix-closed per
 * request and maximise the summed survival score (expected accepted
 * positions).  With B >= sum_r b_r every drafted position is verified (L_r =
 * b_r).  Requires R*b <= 2^24, b <= 64.  Uses the workspace's status word
 * only. */
int32_t dvl_alloc_pack(const float* a, int32_t R, int32_t b, const int32_t* block_len,
                       const int32_t* budget, float* s, int32_t* L, int32_t* pos_off,
                       int32_t* tgt_off, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- row statistics */

/* sv_softmax_stats: per logit row, the largest value, its lowest index and
 * log sum_v exp(l_v / T_r) (computed in double) [DBLast, "What would settle
 * it": target sampling at a temperature].
 *   logits       rows of V values, leading dimension ld (elements)
 *   row_off[R+1] device: work items p in [row_off[r], row_off[r+1]) belong to
 *                request r (an exclusive scan, row_off[0] = 0)
 *   row_stride   host: 0 -> work item p reads logit row p (packed rows);
 *                > 0 -> it reads row r*row_stride + (p - row_off[r]) (dense
 *                rows, e.g. a [R, b, ld] drafter output with row_off = pos_off)
 *   max_rows     host: capacity; row_off[R] <= max_rows
 *   temperature[R]  T_r >= 0; T_r = 0 is greedy (row_lse is then 0)
 *   row_max, row_argmax, row_lse  out: [max_rows], indexed by work item
 * Ties of the maximum go to the lowest index. */
int32_t sv_softmax_stats(const void* logits, int32_t dtype, int64_t ld, int32_t V,
                         const int32_t* row_off, int32_t row_stride, int32_t R, int32_t max_rows,
                         const float* temperature, float* row_max, int32_t* row_argmax,
                         double* row_lse, void* ws, size_t ws_bytes, void* stream);

/* sv_topp_threshold: everything sv_softmax_stats computes, plus the top-p
 * (nucleus) cut [DBLast, "What would settle it": top-p 0.95; reference [18]]:
 *   row_cut       out: the largest logit value t with
 *                 sum_{l_v >= t} softmax(l / T)_v >= top_p_r; every token with
 *                 l_v >= t is kept (ties kept).  -inf when top_p_r >= 1
 *                 (filter off); the row maximum when T_r = 0.
 *   row_kept_lse  out: log sum_{l_v >= cut} exp(l_v / T_r) (double); equals
 *                 row_lse when the filter is off; 0 when T_r = 0.
 * The target probability of token v is then [l_v >= cut] exp(l_v / T -
 * kept_lse).  top_p may be NULL (off for every request).  Same row mapping as
 * sv_softmax_stats. */
int32_t sv_topp_threshold(const void* logits, int32_t dtype, int64_t ld, int32_t V,
                          const int32_t* row_off, int32_t row_stride, int32_t R, int32_t max_rows,
                          const float* temperature, const float* top_p, float* row_max,
                          int32_t* row_argmax, double* row_lse, float* row_cut,
                          double* row_kept_lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- mixture proposal */

/* sv_mixture_q [DBLast, "What carries the argument"; Referee report minor 5,
 * Eq. (20)]: the latent-mixture proposal with greedy branches.
 *   comp_logits  [R, K, b, ld] component logits; branch z of request r at
 *                position i is row (r*K + z)*b + i
 *   mix_logits[R*K]  q(z | y) = softmax over z (float)
 *   pos_off[R+1]     verified positions (from dvl_alloc_pack, or i*b)
 *   max_pos      host: capacity, pos_off[R] <= max_pos
 *   draft_tok[R*b]   the draft block (the branch the drafter decoded)
 *   branch_tok[R*K*b]  out: g_i(z) = argmax_v comp[r, z, i, v] (lowest index),
 *                      written for i < L_r
 *   post_w[R*b*K]    out: category posterior before position i, given the
 *                    draft prefix x_<i: w_z = q(z|y) [g_j(z) = x_j for all
 *                    j < i] / sum of the same over z (double); i < L_r
 *   q_at_draft[R*b]  out: q(x_i | x_<i) = sum of w_z over z with g_i(z) = x_i
 *                    (double); 0 and SV_ST_EMPTY_POSTERIOR when no branch is
 *                    consistent with x_<i; i < L_r
 * Two launches: one block per component row (argmax), then one wave per
 * request (posterior).  Requires K <= 64, b <= 64.  Uses the status word only. */
int32_t sv_mixture_q(const void* comp_logits, int32_t dtype, int64_t ld, int32_t V, int32_t K,
                     int32_t b, const float* mix_logits, const int32_t* pos_off, int32_t R,
                     int32_t max_pos, const int32_t* draft_tok, int32_t* branch_tok,
                     double* post_w, double* q_at_draft, void* ws, size_t ws_bytes,
                     void* stream);

/* sv_verify_rows: sv_topp_threshold over the packed target rows (row_off =
 * tgt_off, row_stride 0) and the branch argmax of sv_mixture_q over the
 * component rows, in ONE launch: its blocks take target rows first and
 * component rows after, so the two read streams share every compute unit.
 * Each component row is streamed by 4 blocks (contiguous quarters); each
 * leaves its partial argmax in the workspace, and sv_accept_sample merges the
 * parts into branch_tok and forms the category posterior.  Arguments as in
 * those two calls (one dtype).  Same method and pages as sv_topp_threshold and
 * sv_mixture_q.
 *   draft_tok[R*b]  the draft tokens (as for sv_accept_sample): the block of
 *                target row j < L_r of request r also keeps the target logit
 *                at draft token j, and every target row's statistics, by
 *                request and position in the workspace, so that the draw of
 *                sv_accept_sample reads them without first reading tgt_off.
 *   branch_T[R]  soft branches [DBLast, "What carries the argument": each
 *                branch is a distribution q_i(. | y, z)], here
 *                softmax(c / T_b,r) (float, device): each component row is
 *                streamed by one block that forms its argmax, maximum and
 *                log sum_v exp(c_v / T_b,r) (fp32 exponentials and partial
 *                sums, double across vectors and threads; fp32 rows: double
 *                throughout); T_b,r = 0 keeps point-mass branches at the
 *                argmax for that request.  NULL: greedy branches for every
 *                request (the four-block partial argmax above).  Pass the
 *                same branch_T to the following sv_accept_sample.
 * Uses the status word and the workspace's branch results: call
 * sv_accept_sample on the same workspace before the next sv_verify_rows. */
int32_t sv_verify_rows(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                       const int32_t* tgt_off, int32_t R, int32_t max_rows, const float* temperature,
                       const float* top_p, float* row_max, int32_t* row_argmax, double* row_lse,
                       float* row_cut, double* row_kept_lse, const void* comp_logits, int64_t comp_ld,
                       int32_t K, int32_t b, const int32_t* pos_off, int32_t max_pos,
                       const int32_t* draft_tok, const float* branch_T, void* ws, size_t ws_bytes,
                       void* stream);

/* sv_verify_rows_dense: sv_topp_threshold over the packed target rows (row_off
 * = tgt_off, row_stride 0) and sv_softmax_stats over the dense draft's rows
 * (row_off = pos_off, row_stride = b: position i of request r is row r*b + i
 * of draft_logits, at the request's temperature, no top-p), in ONE launch:
 * its blocks take target rows first and draft rows after, so both read
 * streams share every compute unit.  Same method and pages as those two calls;
 * outputs as theirs (draft_max, draft_argmax, draft_lse[max_pos] indexed by
 * pos_off[r] + i).  draft_dtype may differ from dtype.  A bf16 row without a
 * cut is streamed in parts by several blocks; the block that finishes a row
 * last merges them (part records and per-row arrival counts in the workspace,
 * the counts back at zero when the call ends).  draft_tok[R*b]: the draft
 * tokens (as for sv_accept_sample); the statistics of every target and draft
 * row, and each row's logit at its draft token, are also kept by request and
 * position in the workspace for the draw of sv_accept_sample.  Uses the
 * workspace's status word, part records and arrival counts. */
int32_t sv_verify_rows_dense(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                             const int32_t* tgt_off, int32_t R, int32_t max_rows, const float* temperature,
                             const float* top_p, float* row_max, int32_t* row_argmax, double* row_lse,
                             float* row_cut, double* row_kept_lse, const void* draft_logits,
                             int32_t draft_dtype, int64_t draft_ld, int32_t b, const int32_t* pos_off,
                             int32_t max_pos, const int32_t* draft_tok, float* draft_max, int32_t* draft_argmax,
                             double* draft_lse, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- acceptance */

/* sv_accept [DBLast, "Assumptions": speculative sampling with rejection
 * correction; reference graph [1], [2]]: for each request and position
 * i = 1..L_r, accept x_i iff u < p_i(x_i) / q_i(x_i | x_<i) (q = 0: accept iff
 * p > 0); n_acc[r] = (first rejected position) - 1, or L_r.
 *   u = (w0 >> 8) * 2^-24, w0 = word 0 of Philox4x32-10 at counter
 *   (i - 1, r, 0, 0) under key (low, high 32 bits of *seed).
 *   Target: row tgt_off[r] + i - 1 of tgt_logits with its row_argmax /
 *   row_cut / row_kept_lse (from sv_topp_threshold; p one-hot at the argmax
 *   when T_r = 0).
 *   q_mode SV_Q_DENSE: draft_logits [R, b, draft_ld]; draft_lse / draft_argmax
 *   indexed by pos_off[r] + i - 1 (from sv_softmax_stats with row_off =
 *   pos_off, row_stride = b); q = exp(d_x / T_r - lse) or one-hot at T_r = 0.
 *   q_mode SV_Q_MIXTURE: q_at_draft[R*b] from sv_mixture_q.
 *   Unused mode's pointers may be NULL.
 *   p_out, q_out (double), u_out (float): optional [R*b] diagnostics.
 * Requires b <= 64.  Uses the workspace's status word only. */
int32_t sv_accept(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                  const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                  const float* temperature, const int32_t* row_argmax, const float* row_cut,
                  const double* row_kept_lse, const int32_t* draft_tok, int32_t q_mode,
                  const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                  const int32_t* draft_argmax, const double* draft_lse,
                  const double* q_at_draft, const uint64_t* seed, int32_t* n_acc,
                  double* p_out, double* q_out, float* u_out, void* ws, size_t ws_bytes,
                  void* stream);

/* ---------------------------------------------------------------- residual / bonus */

/* sv_residual_sample [DBLast, "Assumptions"; reference graph [1], [2]]: one
 * token per request from slot j = n_acc[r] (0-based):
 *   n_acc < L_r: residual norm(max(0, p_j - q_j(. | x_<j))) (if it is zero
 *                everywhere from rounding: p_j);
 *   n_acc = L_r: bonus sample from p_{L_r + 1} (is_bonus = 1).
 *   Inverse CDF in vocabulary order: the smallest v whose running weight
 *   exceeds u * W, u = (w1 >> 8) * 2^-24 from word 1 of Philox at counter
 *   (j, r, 0, 0); weights and their sums in double.  T_r = 0: the argmax.
 *   Arguments as sv_accept; in SV_Q_MIXTURE mode K, branch_tok and post_w
 *   come from sv_mixture_q.
 *   token[R], is_bonus[R]  out.
 * Two launches (sums of the drawn row per 512-value sub-chunk, then the draw);
 * uses the workspace's draw records and sub-chunk sums. */
int32_t sv_residual_sample(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                           const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                           const float* temperature, const int32_t* row_argmax,
                           const float* row_cut, const double* row_kept_lse, int32_t q_mode,
                           const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                           const int32_t* draft_argmax, const double* draft_lse, int32_t K,
                           const int32_t* branch_tok, const double* post_w, const uint64_t* seed,
                           const int32_t* n_acc, int32_t* token, int32_t* is_bonus, void* ws,
                           size_t ws_bytes, void* stream);

/* sv_residual_sample_noalloc: sv_residual_sample for callers that cannot
 * allocate device memory or hand the library a workspace (code under HIP graph
 * capture that must not touch the allocator, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, kernels and results as
 * sv_residual_sample, except that the workspace is replaced by
 *   status      device uint32: the status bits (SV_ST_*) are OR-ed into it
 *               (the caller clears it; it is never reset here)
 * and that the draw records and sub-chunk sums live in a library-owned,
 * fixed-size device array of SV_NOALLOC_SCRATCH_BYTES, one copy per GPU,
 * held until the process ends.  A call needs
 *   round_up_256(1360 * R) + 16 * R * ceil(ceil(V / 8) / 64)  bytes
 * of it (e.g. R <= 128 at V = 151936, R <= 64 at V = 262144); larger problems
 * return SV_ERR_TOO_LARGE before any launch.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's copy of the array, so make the stream's
 * device current.  Calls that overlap on one GPU (other streams, other host
 * threads) share the array and race: serialise them. */
#define SV_NOALLOC_SCRATCH_BYTES (1u << 20)
int32_t sv_residual_sample_noalloc(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                   const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                                   const float* temperature, const int32_t* row_argmax,
                                   const float* row_cut, const double* row_kept_lse, int32_t q_mode,
                                   const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                                   const int32_t* draft_argmax, const double* draft_lse, int32_t K,
                                   const int32_t* branch_tok, const double* post_w, const uint64_t* seed,
                                   const int32_t* n_acc, int32_t* token, int32_t* is_bonus,
                                   uint32_t* status, void* stream);

/* sv_accept_sample: the rest of a step in two launches -- for SV_Q_MIXTURE the
 * branch argmax (merged from the parts sv_verify_rows left in the workspace;
 * branch_tok[R*K*b] out, written for i < L_r) and the category posterior of
 * sv_mixture_q (from mix_logits[R*K] and the draft tokens; writes post_w and
 * q_at_draft), then sv_accept and sv_residual_sample (n_acc, token, is_bonus;
 * optional p_out, q_out, u_out as in sv_accept).  Same method and pages as
 * those calls.  Every chunk block of the draw recomputes its request's
 * posterior and acceptance, so no block waits for another.  With greedy
 * branches or a dense draft the rows' statistics (row_argmax, row_cut,
 * row_kept_lse; draft_argmax, draft_lse) and the logits at the draft tokens
 * are read from the copies the preceding sv_verify_rows or
 * sv_verify_rows_dense left in the workspace (the same values).  SV_Q_DENSE takes
 * the draft arguments of sv_accept; K, mix_logits, branch_tok, post_w,
 * q_at_draft may then be NULL.
 *   branch_T[R], comp_logits, comp_ld  soft branches (NULL: greedy; then
 *                comp_logits may be NULL): the branch statistics come from the
 *                preceding sv_verify_rows with the same branch_T.  The
 *                posterior before position i is proportional to
 *                q(z | y) prod_{j<i} softmax(c_{z,j} / T_b)(x_j) (logs, double);
 *                q(x_i | x_<i) = sum_z w_z softmax(c_{z,i} / T_b)(x_i); the
 *                residual at a rejection j is norm(max(0, p_j - sum_z w_z
 *                softmax(c_{z,j} / T_b))), formed over the K branch rows of
 *                slot j (weights in double).  branch_tok gets each row's
 *                argmax.  Requires K * b <= 2048 and comp_logits in dtype.
 * Uses the workspace's draw records and sub-chunk sums. */
int32_t sv_accept_sample(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                         const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                         const float* temperature, const int32_t* row_argmax, const float* row_cut,
                         const double* row_kept_lse, const int32_t* draft_tok, int32_t q_mode,
                         const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                         const int32_t* draft_argmax, const double* draft_lse, int32_t K,
                         const float* mix_logits, const void* comp_logits, int64_t comp_ld,
                         const float* branch_T, int32_t* branch_tok, double* post_w,
                         double* q_at_draft, const uint64_t* seed, int32_t* n_acc, int32_t* token,
                         int32_t* is_bonus, double* p_out, double* q_out, float* u_out, void* ws,
                         size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- tree verification */

/* Bytes of tree workspace for up to max_nodes tree nodes (all requests), at
 * most max_kids children per node and vocabulary V.  Host-only. */
int32_t sv_tree_workspace_bytes(int32_t max_nodes, int32_t max_kids, int32_t V, size_t* out_bytes);

/* sv_tree_verify: verification of a draft TREE per request [wispaper Q&A on
 * block-diffusion decode failures, section "Why is a fixed block size a
 * failure mode in production?": tree drafters (Bastion; D2SD's prefix trees);
 * rule: multi-round speculative sampling (Miao et al., SpecInfer, ASPLOS
 * 2024), whose rejection correction keeps the target distribution, DBLast
 * review "Assumptions & free parameters"].
 *   node_off[R+1]  exclusive scan of the node counts: request r's nodes are
 *                  k = node_off[r] + j, j = 0 .. N_r - 1 (1 <= N_r <= 1024,
 *                  node_off[R] <= max_nodes); node j = 0 is the root (the
 *                  context so far)
 *   parent[k]      parent of node j, as a local index: -1 for the root, in
 *                  [0, j) otherwise; depth(j) <= b
 *   token[k]       the draft token of node j >= 1
 *   Target rows: row k of tgt_logits is p(. | context, node j's path), with
 *   its statistics row_argmax / row_cut / row_kept_lse[k] (sv_topp_threshold
 *   with row_off = node_off, row_stride 0).
 *   Drafter: the children of a node at depth d were drawn independently from
 *   q_d = softmax(row r*b + d of draft_logits / T_r) (one-hot at its argmax at
 *   T_r = 0), with draft_argmax / draft_lse[r*b + d] (sv_softmax_stats with
 *   row_off = (0, b, 2b, ...), row_stride = b).
 *   Rule, from the root: node u's children, in index order, are tested
 *   against the current target t (first t = p_u): child j with token x is
 *   accepted iff u_j < t(x) / q(x) (q = 0: iff t(x) > 0), u_j from word 0 of
 *   Philox at counter (j - 1, r, 0, 0); on acceptance the walk moves to j
 *   with t = p_j; on rejection t becomes norm(max(0, t - q)) (p_u if that is
 *   empty from rounding); if every child fails, the token is drawn from
 *   norm(max(0, t - q)) of the last rejection; at a node without children a
 *   bonus token is drawn from its p; draws as sv_residual_sample, with word 1
 *   at counter (s, r, 0, 0), s the stopping node.  A chain (parent j - 1) is
 *   exactly sv_accept + sv_residual_sample.  At most max_kids (<= 16)
 *   children per node; at most 1024 requests per call (SV_ERR_ARG beyond).
 *   n_acc[R], path[R*b] (the accepted nodes' local indices in order),
 *   stop_node[R], token_out[R], is_bonus[R]  out
 *   p_out, q_out (double), u_out (float)  optional, [max_nodes] per node: the
 *                  current target's and the draft's probability of the node's
 *                  token and its uniform, for the nodes whose test was reached
 *   ws             workspace of sv_workspace_bytes(R, b, 0, V) (status word,
 *                  draw records, sub-chunk sums)
 *   tree_ws        workspace of sv_tree_workspace_bytes(max_nodes, max_kids, V)
 * Malformed trees (a parent not before its child, depth > b, more than
 * max_kids children, node counts out of range) set SV_ST_BAD_TREE; their
 * request gets n_acc = 0 and no token.  Launches: one block per request
 * (depths, checks, the nodes with several children ordered by their count),
 * max_kids - 1 passes over the (node, 4096-value chunk) items that need them,
 * forming the residual masses sum_v max(0, p - c q), one wave per request
 * (the walk), then the draw's sums and pick. */
int32_t sv_tree_verify(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V, const int32_t* node_off,
                       const int32_t* parent, const int32_t* token, int32_t R, int32_t b, int32_t max_nodes,
                       int32_t max_kids, const float* temperature, const int32_t* row_argmax,
                       const float* row_cut, const double* row_kept_lse, const void* draft_logits,
                       int32_t draft_dtype, int64_t draft_ld, const int32_t* draft_argmax,
                       const double* draft_lse, const uint64_t* seed, int32_t* n_acc, int32_t* path,
                       int32_t* stop_node, int32_t* token_out, int32_t* is_bonus, double* p_out,
                       double* q_out, float* u_out, void* ws, size_t ws_bytes, void* tree_ws,
                       size_t tree_ws_bytes, void* stream);

/* ---------------------------------------------------------------- Philox (test export) */

/* out[(r*n_pos + i)*4 + k] = word k of Philox4x32-10 at counter (i, r, 0, 0)
 * under key (low, high 32 bits of *seed) (Salmon et al., SC'11; the pages
 * name no generator). */
int32_t sv_philox_uniforms(const uint64_t* seed, int32_t R, int32_t n_pos, uint32_t* out,
                           void* stream);

/* Test export: out[k] = exp(x[k]) by the library's table-driven double
 * exponential (the one its probability and draw-weight kernels use; Tang's
 * method, ACM TOMS 1989), for checking its error against the host's exp. */
int32_t sv_selftest_exp(const double* x, double* out, int32_t n, void* stream);

/* Host-only self-checks of code compiled into the library (no GPU needed).
 * sv_selftest_philox_host: the library's Philox4x32-10 round function against
 * the Random123 known-answer vectors (Salmon et al., SC'11).
 * sv_selftest_rows_host: the bf16 value <-> histogram-bin maps and the
 * order-preserving 32-bit float key used by the top-p cut.
 * Each returns 0 on success, else the number of the first failed check. */
int32_t sv_selftest_philox_host(void);
int32_t sv_selftest_rows_host(void);

#ifdef __cplusplus
}
#endif
#endif
