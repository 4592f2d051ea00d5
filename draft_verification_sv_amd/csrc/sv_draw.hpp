// sv_draw.hpp -- row loads (16-byte groups of 8 values) and the arguments of
// the acceptance and draw kernels (sv_sample.hip), shared with the tree
// verification, which prepares draw records of its own and has them summed
// and picked by the same kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv_device.hpp"

namespace sv {

__device__ __forceinline__ const char* row_ptr(const void* base, int dtype, int64_t row, int64_t ld) {
  return static_cast<const char*>(base) + static_cast<size_t>(row) * static_cast<size_t>(ld) * (dtype == SV_BF16 ? 2 : 4);
}

// The 8 values of group g (elements 8g .. 8g+7) as raw 16-byte words, issued
// before any of them is used so that all of a thread's loads are in flight
// together; decode8 converts them and reads elements >= V (and every element
// of a group that is not `in` the row) as -inf.  Row bases
// and pitches are 16-byte multiples, so an aligned 16-byte word holding an
// element below V lies in the same mapped page as that element; the fp32 upper
// word is read only when it holds one (else the lower word is read twice).
template <int DT>
__device__ __forceinline__ void raw8(const char* rowp, int g, int V, uint4& w0, uint4& w1) {
  if constexpr (DT == SV_BF16) {
    w0 = *reinterpret_cast<const uint4*>(rowp + static_cast<size_t>(g) * 16);
    w1 = w0;
  } else {
    const char* q = rowp + static_cast<size_t>(g) * 32;
    w0 = *reinterpret_cast<const uint4*>(q);
    w1 = *reinterpret_cast<const uint4*>(g * 8 + 4 < V ? q + 16 : q);
  }
}

template <int DT>
__device__ __forceinline__ void decode8(const uint4& w0, const uint4& w1, int g, int V, bool in, float out[8]) {
  float v[8];
  if constexpr (DT == SV_BF16) {
    v[0] = bf16_lo(w0.x); v[1] = bf16_hi(w0.x); v[2] = bf16_lo(w0.y); v[3] = bf16_hi(w0.y);
    v[4] = bf16_lo(w0.z); v[5] = bf16_hi(w0.z); v[6] = bf16_lo(w0.w); v[7] = bf16_hi(w0.w);
  } else {
    v[0] = __uint_as_float(w0.x); v[1] = __uint_as_float(w0.y); v[2] = __uint_as_float(w0.z); v[3] = __uint_as_float(w0.w);
    v[4] = __uint_as_float(w1.x); v[5] = __uint_as_float(w1.y); v[6] = __uint_as_float(w1.z); v[7] = __uint_as_float(w1.w);
  }
  const int valid = in ? min(max(V - g * 8, 0), 8) : 0;  // elements of the group below V
#pragma unroll
  for (int k = 0; k < 8; ++k) out[k] = k < valid ? v[k] : -INFINITY;
}

// The 8 values of a group from its raw words, unmasked.
template <int DT>
__device__ __forceinline__ void unpack8(const uint4& w0, const uint4& w1, float v[8]) {
  if constexpr (DT == SV_BF16) {
    v[0] = bf16_lo(w0.x); v[1] = bf16_hi(w0.x); v[2] = bf16_lo(w0.y); v[3] = bf16_hi(w0.y);
    v[4] = bf16_lo(w0.z); v[5] = bf16_hi(w0.z); v[6] = bf16_lo(w0.w); v[7] = bf16_hi(w0.w);
  } else {
    v[0] = __uint_as_float(w0.x); v[1] = __uint_as_float(w0.y); v[2] = __uint_as_float(w0.z); v[3] = __uint_as_float(w0.w);
    v[4] = __uint_as_float(w1.x); v[5] = __uint_as_float(w1.y); v[6] = __uint_as_float(w1.z); v[7] = __uint_as_float(w1.w);
  }
}

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
  const SlotRec* slot;        // fused tail: the rows launch's statistics by (request, row)
  const SlotRec* dslot;       // fused dense tail: the draft rows' lse, argmax and x logit by (request, position)
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
