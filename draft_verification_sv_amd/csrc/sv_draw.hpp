// sv_draw.hpp -- arguments of the acceptance and draw kernels (sv_sample.hip),
// shared with the tree verification, which prepares draw records of its own
// and has them summed and picked by the same kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.hpp"

namespace sv {

struct SampleArgs {
  const void* tgt;
  int dtype;
  int64_t tgt_ld;
  int V;
  const int32_t* tgt_off;
  const int32_t* pos_off;
  int R, b;
  const float* T;
  const int32_t* row_argmax;
  const float* row_cut;
  const double* row_kept;
  const int32_t* x;
  int q_mode;
  const void* draft;
  int ddtype;
  int64_t draft_ld;
  const int32_t* dargmax;
  const double* dlse;
  const double* qx;  // q at the draft tokens (mixture, standalone acceptance)
  int K;
  const float* mix;  // mixing logits (fused tail)
  const int32_t* branch_tok;  // standalone draw: the branch argmax
  const uint64_t* bkey;       // fused tail: the partial argmax keys of the rows launch
  int32_t* branch_out;        // fused tail: the branch argmax, written for i < L_r
  double* post_w;      // read by the standalone draw; written by the fused tail
  double* q_at_draft;  // written by the fused tail
  const uint64_t* seed;
  const int32_t* n_acc_in;
  int32_t* n_acc;
  int32_t* token;
  int32_t* is_bonus;
  double* p_out;
  double* q_out;
  float* u_out;
  DrawRec* rec;  // [R] draw records
  double* sub;   // [R * NSUB * 2] sub-chunk sums {draw weight, p}
  int NSUB;      // sub-chunks per row
  int S;         // chunks per row
  uint32_t* status;
  const void* comp;        // soft branches: component rows [R*K*b, comp_ld], target dtype
  int64_t comp_ld;
  const float* branch_T;   // soft branches: T_b per request
  const double* blse;      // soft branches: lse(c / T_b) per component row (rows launch)
  const int32_t* barg;     // soft branches: argmax per component row (rows launch)
};

// Sums and pick of one draw per request from the records the caller's kernels
// left in a.rec (mode, drawn row, cut, kept mass, 1/T, the dense draft row and
// its log-normaliser; SV_Q_DENSE weights max(0, p - exp(d / T - dlse))).
// Defined in sv_sample.hip.
int32_t launch_record_draw(const SampleArgs& a, hipStream_t s);

}  // namespace sv
