// sv_mix.hip -- latent-mixture proposal: branch statistics and the category
// posterior.
//
// "Pith review of DBLAST", "What carries the argument": the block proposal is
// q_dep(x_1:b | y) = sum_z q(z|y) prod_i q_i(x_i | y, z).  The drafter draws
// one category and emits that branch's argmax tokens; the verifier scores each
// position under the mixture whose category weights have been updated by the
// draft prefix (the greedy-branch conditional, Eq. (20) per the Referee
// report, minor 5).  With
// point-mass branches at g_i(z) = argmax_v c_{r,z,i,v}, the posterior before
// position i keeps the categories whose branch agrees with the draft prefix:
//   w_z = q(z|y) [g_j(z) = x_j, j < i] / sum over z of the same,
//   q(x_i | x_<i) = sum of w_z over z with g_i(z) = x_i.
//
// k_mix_argmax: one 256-thread block per component row (position, category)
// streams the row once with 128-bit non-temporal loads, two batches of four
// 16-byte loads in flight per thread (double-buffered; 49 VGPRs keeps eight
// waves per SIMD, so every row of a step is resident at once), keeps the maximum of every 8-value
// vector and the winning vector, and reduces (value, lowest index) over the
// wave and the block.  One block per row needs no cross-block merge.
// k_mix_post: one wave per request runs the posterior recursion over the
// positions with one lane per category (K <= 64), in double.
//
// Soft branches (same review, "What carries the argument": each branch is a
// distribution q_i(. | y, z); here softmax(c / T_b)): the fused rows launch
// gives every component row one block that forms lse(c / T_b), argmax and
// maximum in one streaming pass (stream_row_bf16); the draw kernels form the
// posterior from them (sv_sample.hip).
#include <math.h>

#include "sv_device.hpp"
#include "sv_host.hpp"
#include "sv_rows_dev.hpp"

namespace sv {

constexpr int kMixNT = 256;
constexpr int kMixBatch = 4;  // 16-byte loads per thread per batch (x2 in flight)

struct MixArgs {
  const void* comp;
  int64_t ld;
  int V, K, b;
  const float* mix;
  const int32_t* pos_off;
  int R, max_pos;
  const int32_t* x;
  int32_t* branch_tok;  // the argmax (one block per row), or
  uint64_t* bkey;       // the partial argmax keys of `parts` blocks per row
  int parts;
  double* post_w;
  double* q;
  uint32_t* status;
  const float* branch_T;  // soft branches: temperature per request (device), else NULL
  double* blse;           // soft branches: lse of c / T_b per component row [R*K*b]
  int32_t* barg;          // soft branches: argmax per component row
  float* bmax;            // soft branches: maximum per component row
};

// Order-preserving key of a float with -0 folded onto +0.
__device__ __forceinline__ uint32_t fkey(float f) {
  f = f + 0.0f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <int DT>
__device__ __forceinline__ float vec_max(const uint4& d) {
  if constexpr (DT == SV_BF16) {
    return fmaxf(fmaxf(fmaxf(bf16_lo(d.x), bf16_hi(d.x)), fmaxf(bf16_lo(d.y), bf16_hi(d.y))),
                 fmaxf(fmaxf(bf16_lo(d.z), bf16_hi(d.z)), fmaxf(bf16_lo(d.w), bf16_hi(d.w))));
  } else {
    return fmaxf(fmaxf(__uint_as_float(d.x), __uint_as_float(d.y)), fmaxf(__uint_as_float(d.z), __uint_as_float(d.w)));
  }
}

// Largest magnitude field of a vector's values (sign bits cleared), per 16-bit
// half for bf16 (two halves) and per word for fp32: a value is +-inf or NaN iff
// its magnitude reaches the all-ones exponent (0x7F80 / 0x7F800000).
template <int DT>
__device__ __forceinline__ uint32_t vec_mag(const uint4& d) {
  if constexpr (DT == SV_BF16) {
    constexpr uint32_t m = 0x7FFF7FFFu;
    return __builtin_bit_cast(
        uint32_t, __builtin_elementwise_max(
                      __builtin_elementwise_max(__builtin_bit_cast(u16x2, d.x & m), __builtin_bit_cast(u16x2, d.y & m)),
                      __builtin_elementwise_max(__builtin_bit_cast(u16x2, d.z & m), __builtin_bit_cast(u16x2, d.w & m))));
  } else {
    constexpr uint32_t m = 0x7FFFFFFFu;
    return max(max(d.x & m, d.y & m), max(d.z & m, d.w & m));
  }
}

template <int DT>
__device__ __forceinline__ uint32_t mag_max(uint32_t a, uint32_t b) {
  if constexpr (DT == SV_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
  else
    return max(a, b);
}

template <int DT>
__device__ __forceinline__ bool mag_nonfinite(uint32_t m) {
  if constexpr (DT == SV_BF16)
    return (m & 0xFFFFu) >= 0x7F80u || (m >> 16) >= 0x7F80u;
  else
    return m >= 0x7F800000u;
}

// Streams vectors [v0, v1) of a row with stride NT per thread; returns the
// thread's best (value, element index) with the lowest index among ties, or
// index -1 if it saw no vector, and whether one of its values was +-inf or NaN.
template <int DT, int NT>
__device__ __forceinline__ void stream_argmax(const uint4* vp, int v0, int v1, float& best, int& bidx,
                                              bool& nonfinite) {
  constexpr int PER = DT == SV_BF16 ? 8 : 4;
  uint32_t mg = 0;
  best = -INFINITY;
  int bvi = -1;
  uint4 bv = {0, 0, 0, 0};
  int v = v0 + static_cast<int>(threadIdx.x);
  // loads are unconditional, their indices clamped to the range's last vector
  // (re-read, unused), so that no branch makes the compiler wait for the batch
  // in flight before using the one before it
  const int last = v1 - 1;
  uint4 cur[kMixBatch];
  if (v1 > v0) {
#pragma unroll
    for (int k = 0; k < kMixBatch; ++k) cur[k] = load16_stream(vp + min(v + k * NT, last));
  }
  while (v < v1) {
    const int vn = v + kMixBatch * NT;
    uint4 nxt[kMixBatch];
#pragma unroll
    for (int k = 0; k < kMixBatch; ++k) nxt[k] = load16_stream(vp + min(vn + k * NT, last));
#pragma unroll
    for (int k = 0; k < kMixBatch; ++k) {
      if (v + k * NT < v1) {
        const float m = vec_max<DT>(cur[k]);
        mg = mag_max<DT>(mg, vec_mag<DT>(cur[k]));
        if (m > best) {
          best = m;
          bvi = v + k * NT;
          bv = cur[k];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kMixBatch; ++k) cur[k] = nxt[k];
    v = vn;
  }
  bidx = -1;
  if (bvi >= 0) {
    float e[PER];
    if constexpr (DT == SV_BF16) {
      e[0] = bf16_lo(bv.x); e[1] = bf16_hi(bv.x); e[2] = bf16_lo(bv.y); e[3] = bf16_hi(bv.y);
      e[4] = bf16_lo(bv.z); e[5] = bf16_hi(bv.z); e[6] = bf16_lo(bv.w); e[7] = bf16_hi(bv.w);
    } else {
      e[0] = __uint_as_float(bv.x); e[1] = __uint_as_float(bv.y); e[2] = __uint_as_float(bv.z); e[3] = __uint_as_float(bv.w);
    }
    int k = PER - 1;
#pragma unroll
    for (int q = PER - 1; q >= 0; --q)
      if (e[q] == best) k = q;
    bidx = bvi * PER + k;
  }
  nonfinite = mag_nonfinite<DT>(mg);
}

// argmax of part `part` (of a.parts) of component row m = p*K + z (position p,
// category z) by one block
template <int DT, int NT>
__device__ __forceinline__ void mix_block(const MixArgs& a, int m, int part, uint64_t* red, int* s_req) {
  const int tid = threadIdx.x;
  const int z = m % a.K;
  const int p = m / a.K;
  const int total = a.pos_off[a.R];
  if (m == 0 && tid == 0 && (a.pos_off[0] != 0 || total > a.max_pos || total < 0))
    raise_status(a.status, SV_ST_BAD_OFFSETS);
  if (p >= total) return;
  const int r = find_request<NT>(a.pos_off, a.R, p, s_req);
  if (r < 0) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  const int i = p - a.pos_off[r];
  if (i >= a.b) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  constexpr int PER = DT == SV_BF16 ? 8 : 4;
  const size_t esz = DT == SV_BF16 ? 2 : 4;
  const int64_t row = (static_cast<int64_t>(r) * a.K + z) * a.b + i;
  const char* rowp = static_cast<const char*>(a.comp) + static_cast<size_t>(row) * static_cast<size_t>(a.ld) * esz;
  const int nvec = a.V / PER;
  const int v0 = static_cast<int>(static_cast<int64_t>(nvec) * part / a.parts);
  const int v1 = static_cast<int>(static_cast<int64_t>(nvec) * (part + 1) / a.parts);
  float best;
  int bidx;
  bool nonfinite;
  stream_argmax<DT, NT>(reinterpret_cast<const uint4*>(rowp), v0, v1, best, bidx, nonfinite);
  if (part == a.parts - 1)
    for (int e = nvec * PER + tid; e < a.V; e += NT) {  // elements past the last full vector
      const float f = load_val<DT>(rowp, e);
      nonfinite |= !isfinite(f);
      if (f > best || bidx < 0) {
        best = f;
        bidx = e;
      }
    }
  if (nonfinite) raise_status(a.status, SV_ST_NONFINITE);
  uint64_t packed = bidx >= 0 ? (static_cast<uint64_t>(fkey(best)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bidx)) : 0;
  packed = block_max_u64<NT>(packed, red);
  if (tid == 0) {
    const size_t slot = (static_cast<size_t>(r) * a.K + z) * a.b + i;
    if (a.bkey)
      a.bkey[slot * a.parts + part] = packed;
    else
      a.branch_tok[slot] = static_cast<int>(argmax_token(packed));
  }
}

// Soft branches: statistics of component row m = p*K + z (position p, category
// z) at its request's branch temperature T_b, by one block: lse of c / T_b,
// argmax and maximum (T_b = 0: argmax and maximum), with the row statistics'
// code without a cut (bf16: one streaming pass; fp32: the generic path).
template <int DT, int NT, int BATCH>
__device__ __forceinline__ void soft_block(const MixArgs& a, int m, uint32_t* hist, RowShared<NT>& sh) {
  const int tid = threadIdx.x;
  const int z = m % a.K;
  const int p = m / a.K;
  const int total = a.pos_off[a.R];
  if (m == 0 && tid == 0 && (a.pos_off[0] != 0 || total > a.max_pos || total < 0))
    raise_status(a.status, SV_ST_BAD_OFFSETS);
  if (p >= total) return;
  const int r = find_request<NT>(a.pos_off, a.R, p, &sh.req);
  if (r < 0) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  const int i = p - a.pos_off[r];
  if (i >= a.b) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  const size_t esz = DT == SV_BF16 ? 2 : 4;
  const int64_t row = (static_cast<int64_t>(r) * a.K + z) * a.b + i;
  const char* rowp = static_cast<const char*>(a.comp) + static_cast<size_t>(row) * static_cast<size_t>(a.ld) * esz;
  const float Tb = a.branch_T[r];
  if (tid == 0 && !(Tb >= 0.0f)) raise_status(a.status, SV_ST_BAD_TEMPERATURE);
  RowArgs ca{};
  ca.logits = a.comp;
  ca.ld = a.ld;
  ca.V = a.V;
  ca.R = a.R;
  ca.row_max = a.bmax;
  ca.row_argmax = a.barg;
  ca.row_lse = a.blse;
  ca.status = a.status;
  row_stats_at<DT, NT, BATCH>(ca, rowp, static_cast<int>(row), Tb, 1.0f, false, hist, sh);
}

template <int DT>
__global__ __launch_bounds__(kMixNT) void k_mix_argmax(MixArgs a) {
  __shared__ uint64_t red[kMixNT / kWave];
  __shared__ int s_req;
  mix_block<DT, kMixNT>(a, blockIdx.x, 0, red, &s_req);
}

// One launch for the target rows and the component rows of a step: blocks
// [0, n_row_blocks) take target rows (statistics and top-p cut), the rest take
// one kMixParts-th of a component row each (partial branch argmax).  Lower
// block numbers are dispatched first, so the target rows, which carry more work
// per byte, start at once on every CU and share it with the component
// streaming.  The launch has more blocks than fit at once; short component
// blocks keep the last round short (32 requests with DVL 256, K = 8 and
// V = 151936: 107 us with 4 parts per row against 110 us with whole rows).
constexpr int kFusedNT = 256;
constexpr int kFusedBatch = 4;

template <int DT, bool kSoft>
__global__ __launch_bounds__(kFusedNT) void k_rows_mix(RowArgs ra, MixArgs ma, int n_row_blocks) {
  __shared__ RowShared<kFusedNT> sh;
  __shared__ uint32_t hist[DT == SV_BF16 ? kHistWords : 1];
  const int blk = blockIdx.x;
  if (blk < n_row_blocks) {
    const int total = ra.row_off[ra.R];
    if (blk == 0 && threadIdx.x == 0 && (ra.row_off[0] != 0 || total > ra.max_rows || total < 0))
      raise_status(ra.status, SV_ST_BAD_OFFSETS);
    if (blk >= total) return;
    exp_table_init(sh.etab);  // published by row_block's first barrier
    row_block<DT, kFusedNT, kFusedBatch, kSoft>(ra, blk, hist, sh);  // the greedy kernel keeps its register budget
  } else {
    const int u = blk - n_row_blocks;
    if constexpr (kSoft)
      soft_block<DT, kFusedNT, kFusedBatch>(ma, u, hist, sh);
    else
      mix_block<DT, kFusedNT>(ma, u / kMixParts, u % kMixParts, sh.red_u64, &sh.req);
  }
}

__global__ __launch_bounds__(kWave) void k_mix_post(MixArgs a) {
  __shared__ int gtab[64 * 64];  // branch tokens of this request, [z][i]
  __shared__ int xtab[64];
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const int base = a.pos_off[r];
  const int Lr = a.pos_off[r + 1] - base;
  if (Lr < 0 || Lr > a.b || a.pos_off[a.R] > a.max_pos) return;  // reported by k_mix_argmax
  // all loads first: the recursion below then runs out of LDS and registers
  for (int k = lane; k < a.K * Lr; k += kWave) {
    const int zz = k / Lr, ii = k % Lr;
    gtab[zz * 64 + ii] = a.branch_tok[(static_cast<size_t>(r) * a.K + zz) * a.b + ii];
  }
  if (lane < Lr) xtab[lane] = a.x[static_cast<size_t>(r) * a.b + lane];
  const bool act = lane < a.K;
  const float ml = act ? a.mix[static_cast<size_t>(r) * a.K + lane] : -INFINITY;
  __syncthreads();
  const float mmax = wave_max_f32(ml);
  const double e = act ? exp(static_cast<double>(ml) - static_cast<double>(mmax)) : 0.0;
  const double pi = e / wave_sum_f64(e);  // q(z | y)
  bool consistent = act;
  for (int ii = 0; ii < Lr; ++ii) {
    const int g = act ? gtab[lane * 64 + ii] : -1;
    const double w = consistent ? pi : 0.0;
    const double sw = wave_sum_f64(w);
    const double post = sw > 0.0 ? w / sw : 0.0;
    if (act) a.post_w[(static_cast<size_t>(r) * a.b + ii) * a.K + lane] = post;
    const int xi = xtab[ii];
    const double qsum = wave_sum_f64(act && g == xi ? post : 0.0);
    if (lane == 0) {
      a.q[static_cast<size_t>(r) * a.b + ii] = qsum;
      if (!(sw > 0.0)) raise_status(a.status, SV_ST_EMPTY_POSTERIOR);
      if (xi < 0 || xi >= a.V) raise_status(a.status, SV_ST_BAD_TOKEN);
    }
    consistent = consistent && (g == xi);
  }
}

}  // namespace sv

using namespace sv;

static bool mix_args_ok(const void* comp_logits, int32_t dtype, int64_t ld, int32_t V, int32_t K, int32_t b,
                        const float* mix_logits, const int32_t* pos_off, int32_t R, int32_t max_pos,
                        const int32_t* draft_tok, int32_t* branch_tok, double* post_w, double* q_at_draft, void* ws) {
  if (!comp_logits || !mix_logits || !pos_off || !draft_tok || !branch_tok || !post_w || !q_at_draft || !ws)
    return false;
  if (R < 1 || V < 1 || K < 1 || K > 64 || b < 1 || b > 64 || ld < V || max_pos < 0) return false;
  if (dtype != SV_F32 && dtype != SV_BF16) return false;
  if (!rows_aligned(comp_logits, dtype, ld)) return false;
  if (static_cast<long long>(max_pos) > static_cast<long long>(R) * b) return false;
  if (static_cast<long long>(max_pos) * K > 0x3FFFFFFFLL) return false;
  return true;
}

extern "C" int32_t sv_mixture_q(const void* comp_logits, int32_t dtype, int64_t ld, int32_t V, int32_t K, int32_t b,
                                const float* mix_logits, const int32_t* pos_off, int32_t R, int32_t max_pos,
                                const int32_t* draft_tok, int32_t* branch_tok, double* post_w, double* q_at_draft,
                                void* ws, size_t ws_bytes, void* stream) {
  if (!mix_args_ok(comp_logits, dtype, ld, V, K, b, mix_logits, pos_off, R, max_pos, draft_tok, branch_tok, post_w,
                   q_at_draft, ws))
    return SV_ERR_ARG;
  if (ws_bytes < ws_layout(R, b, K, V).total) return SV_ERR_WORKSPACE;
  if (max_pos == 0) return SV_OK;
  MixArgs a{comp_logits, ld, V, K, b, mix_logits, pos_off, R, max_pos, draft_tok, branch_tok, nullptr, 1,
            post_w, q_at_draft, status_word(ws)};
  const long long grid = static_cast<long long>(max_pos) * K;
  if (grid > 0x7FFFFFFFLL) return SV_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(k_mix_argmax<SV_BF16>, dim3(static_cast<unsigned>(grid)), dim3(kMixNT), 0, s, a);
  else
    hipLaunchKernelGGL(k_mix_argmax<SV_F32>, dim3(static_cast<unsigned>(grid)), dim3(kMixNT), 0, s, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  hipLaunchKernelGGL(k_mix_post, dim3(R), dim3(kWave), 0, s, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_verify_rows(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                  const int32_t* tgt_off, int32_t R, int32_t max_rows, const float* temperature,
                                  const float* top_p, float* row_max, int32_t* row_argmax, double* row_lse,
                                  float* row_cut, double* row_kept_lse, const void* comp_logits, int64_t comp_ld,
                                  int32_t K, int32_t b, const int32_t* pos_off, int32_t max_pos,
                                  const int32_t* draft_tok, const float* branch_T, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!tgt_logits || !tgt_off || !temperature || !row_max || !row_argmax || !row_lse || !row_cut || !row_kept_lse)
    return SV_ERR_ARG;
  if (!comp_logits || !pos_off || !draft_tok || !ws) return SV_ERR_ARG;
  if (R < 1 || V < 1 || K < 1 || K > 64 || b < 1 || b > 64 || max_rows < 0 || max_pos < 0) return SV_ERR_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_ARG;
  if (tgt_ld < V || comp_ld < V || !rows_aligned(tgt_logits, dtype, tgt_ld) || !rows_aligned(comp_logits, dtype, comp_ld))
    return SV_ERR_ARG;
  if (static_cast<long long>(max_pos) > static_cast<long long>(R) * b) return SV_ERR_ARG;
  if (static_cast<long long>(max_rows) + static_cast<long long>(max_pos) * K * kMixParts > 0x7FFFFFFFLL)
    return SV_ERR_ARG;
  const WsLayout l = ws_layout(R, b, K, V);
  if (ws_bytes < l.total) return SV_ERR_WORKSPACE;
  RowArgs ra{tgt_logits, tgt_ld, V, tgt_off, 0, R, max_rows, temperature, top_p, row_max, row_argmax, row_lse,
             row_cut, row_kept_lse, status_word(ws)};
  ra.slot = reinterpret_cast<SlotRec*>(static_cast<char*>(ws) + l.slot);
  ra.gx = draft_tok;
  ra.slot_b = b;
  MixArgs ma{comp_logits, comp_ld, V, K, b, nullptr, pos_off, R, max_pos, nullptr, nullptr,
             reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + l.bkey), kMixParts, nullptr, nullptr,
             status_word(ws)};
  const bool soft = branch_T != nullptr;
  if (soft) {
    ma.branch_T = branch_T;
    ma.blse = reinterpret_cast<double*>(static_cast<char*>(ws) + l.blse);
    ma.barg = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + l.barg);
    ma.bmax = reinterpret_cast<float*>(static_cast<char*>(ws) + l.bmax);
  }
  // greedy branches: kMixParts blocks per component row; soft: one
  const unsigned mix_blocks = static_cast<unsigned>(max_pos) * static_cast<unsigned>(K) * (soft ? 1u : kMixParts);
  const unsigned grid = static_cast<unsigned>(max_rows) + mix_blocks;
  if (grid == 0) return SV_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == SV_BF16) {
    if (soft)
      hipLaunchKernelGGL((k_rows_mix<SV_BF16, true>), dim3(grid), dim3(kFusedNT), 0, s, ra, ma, max_rows);
    else
      hipLaunchKernelGGL((k_rows_mix<SV_BF16, false>), dim3(grid), dim3(kFusedNT), 0, s, ra, ma, max_rows);
  } else {
    if (soft)
      hipLaunchKernelGGL((k_rows_mix<SV_F32, true>), dim3(grid), dim3(kFusedNT), 0, s, ra, ma, max_rows);
    else
      hipLaunchKernelGGL((k_rows_mix<SV_F32, false>), dim3(grid), dim3(kFusedNT), 0, s, ra, ma, max_rows);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
