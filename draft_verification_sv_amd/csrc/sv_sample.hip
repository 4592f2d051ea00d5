// sv_sample.hip -- acceptance tests, first rejection, residual and bonus samples.
//
// Speculative sampling with rejection correction ("Pith review of DBLAST",
// "Assumptions & free parameters"; reference graph [1] Leviathan et al., [2]
// Chen et al.): position i of request r is accepted iff u < p_i(x_i) / q_i(x_i |
// x_<i); the first rejection at position j ends the block and one token is
// drawn from norm(max(0, p_j - q_j)); when all L_r positions pass, a bonus token
// is drawn from p_{L_r + 1}.  Uniforms come from Philox4x32-10 at counter
// (position, request, 0, 0): word 0 for the test, word 1 for the draw.
//
// k_accept: one wave per request, one lane per position (b <= 64); p and q at
// the draft token are gathered and compared in double; a ballot over the
// rejecting lanes gives the first rejection.
// The sampled row of each request is cut into S <= 64 chunks.  k_res_sums: one
// wave per chunk forms the weights of its chunk in double and stores their sum
// (and the sum of p).  k_res_pick (after a kernel boundary): one wave per
// request scans the chunk sums (one per lane) to find the chunk holding u * W,
// then walks that chunk 512 values at a time: per-lane sums of 8 consecutive
// weights, a shuffle scan across the wave, and a ballot for the first lane
// whose running weight exceeds u * W.
#include <math.h>

#include "sv_device.hpp"
#include "sv_host.hpp"

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
  const double* qx;  // accept, mixture mode
  int K;             // residual, mixture mode
  const int32_t* branch_tok;
  const double* post_w;
  const uint64_t* seed;
  const int32_t* n_acc_in;
  int32_t* n_acc;
  int32_t* token;
  int32_t* is_bonus;
  double* p_out;
  double* q_out;
  float* u_out;
  double* part;        // [R * S * 2] chunk sums (residual)
  int S;               // chunks per row (residual)
  int CG;              // 8-element groups per chunk (residual)
  uint32_t* status;
};

__device__ __forceinline__ const char* row_ptr(const void* base, int dtype, int64_t row, int64_t ld) {
  return static_cast<const char*>(base) + static_cast<size_t>(row) * static_cast<size_t>(ld) * (dtype == SV_BF16 ? 2 : 4);
}

// target probability of token v: [l >= cut] exp(l / T - kept_lse), T > 0
__device__ __forceinline__ double p_of(float l, float cut, double Td, double kept) {
  return l >= cut ? exp(static_cast<double>(l) / Td - kept) : 0.0;
}

// ------------------------------------------------------------------ acceptance
__global__ __launch_bounds__(kWave) void k_accept(SampleArgs a) {
  const int r = blockIdx.x;
  const int i = threadIdx.x;
  const int pb = a.pos_off[r];
  const int Lr = a.pos_off[r + 1] - pb;
  const int tb = a.tgt_off[r];
  const bool offs_ok = Lr >= 0 && Lr <= a.b && a.tgt_off[r + 1] - tb == Lr + 1;
  if (!offs_ok) {
    if (i == 0) {
      raise_status(a.status, SV_ST_BAD_OFFSETS);
      a.n_acc[r] = 0;
    }
    return;
  }
  const uint64_t seed = *a.seed;
  const float T = a.T[r];
  bool reject = false;
  if (i < Lr) {
    const int xv = a.x[static_cast<size_t>(r) * a.b + i];
    const bool tok_ok = xv >= 0 && xv < a.V;
    if (!tok_ok) raise_status(a.status, SV_ST_BAD_TOKEN);
    const int trow = tb + i;
    double p = 0.0, q = 0.0;
    if (tok_ok) {
      if (T == 0.0f) {
        p = xv == a.row_argmax[trow] ? 1.0 : 0.0;
      } else {
        const float l = load_val_rt(row_ptr(a.tgt, a.dtype, trow, a.tgt_ld), a.dtype, xv);
        p = p_of(l, a.row_cut[trow], static_cast<double>(T), a.row_kept[trow]);
      }
      if (a.q_mode == SV_Q_MIXTURE) {
        q = a.qx[static_cast<size_t>(r) * a.b + i];
      } else {
        const int pos = pb + i;
        if (T == 0.0f) {
          q = xv == a.dargmax[pos] ? 1.0 : 0.0;
        } else {
          const float d = load_val_rt(row_ptr(a.draft, a.ddtype, static_cast<int64_t>(r) * a.b + i, a.draft_ld), a.ddtype, xv);
          q = exp(static_cast<double>(d) / static_cast<double>(T) - a.dlse[pos]);
        }
      }
    }
    const U4 w = philox_at(seed, static_cast<uint32_t>(i), static_cast<uint32_t>(r));
    const double u = u24(w.x);
    const bool accept = q > 0.0 ? (u < p / q) : (p > 0.0);
    reject = !accept;
    const size_t k = static_cast<size_t>(r) * a.b + i;
    if (a.p_out) a.p_out[k] = p;
    if (a.q_out) a.q_out[k] = q;
    if (a.u_out) a.u_out[k] = static_cast<float>(u);
  }
  const uint64_t mask = __ballot(reject);
  if (i == 0) a.n_acc[r] = mask ? (__ffsll(static_cast<long long>(mask)) - 1) : Lr;
}

// ------------------------------------------------------------------ residual / bonus
// One wave per block.  A chunk is a run of 8-value groups; lane l takes groups
// l, l + 64, l + 128, ... so every load instruction of the wave reads 1 KiB of
// consecutive logits, and 64 consecutive groups form a "row" of 512 values that
// the wave scans with shuffles.
constexpr int kResChunks = 64;

// 8 consecutive values starting at element 8g (elements >= V read as -inf)
__device__ __forceinline__ void load8(const char* rowp, int dtype, int g, int V, float out[8]) {
  const int e0 = g * 8;
  if (e0 + 8 <= V) {
    if (dtype == SV_BF16) {
      const uint4 d = *reinterpret_cast<const uint4*>(rowp + static_cast<size_t>(e0) * 2);
      out[0] = bf16_lo(d.x); out[1] = bf16_hi(d.x); out[2] = bf16_lo(d.y); out[3] = bf16_hi(d.y);
      out[4] = bf16_lo(d.z); out[5] = bf16_hi(d.z); out[6] = bf16_lo(d.w); out[7] = bf16_hi(d.w);
    } else {
      const uint4 d0 = *reinterpret_cast<const uint4*>(rowp + static_cast<size_t>(e0) * 4);
      const uint4 d1 = *reinterpret_cast<const uint4*>(rowp + static_cast<size_t>(e0) * 4 + 16);
      out[0] = __uint_as_float(d0.x); out[1] = __uint_as_float(d0.y); out[2] = __uint_as_float(d0.z); out[3] = __uint_as_float(d0.w);
      out[4] = __uint_as_float(d1.x); out[5] = __uint_as_float(d1.y); out[6] = __uint_as_float(d1.z); out[7] = __uint_as_float(d1.w);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = e0 + k < V ? load_val_rt(rowp, dtype, e0 + k) : -INFINITY;
  }
}

// What one request's draw needs; filled by res_setup.
struct ResCtx {
  int j, trow;
  bool bonus;
  double Td, kept, dlse;
  float cut;
  const char* trowp;
  const char* drowp;
  int nq;        // mixture: branch entries at slot j (K, with their posterior mass)
  int qtok[64];  // kept in LDS
  double qw[64];
};

// Returns false when the request needs no scan (T = 0: the draw is the argmax,
// written here by the reporting kernel).
template <bool kDense>
__device__ __forceinline__ bool res_setup(const SampleArgs& a, int r, bool report, ResCtx& c) {
  const int lane = threadIdx.x;
  const int pb = a.pos_off[r];
  const int Lr = a.pos_off[r + 1] - pb;
  const int tb = a.tgt_off[r];
  if (!(Lr >= 0 && Lr <= a.b && a.tgt_off[r + 1] - tb == Lr + 1)) {
    if (report && lane == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return false;
  }
  int n = a.n_acc_in[r];
  if (n < 0 || n > Lr) {
    if (report && lane == 0) raise_status(a.status, SV_ST_BAD_NACC);
    n = n < 0 ? 0 : Lr;
  }
  c.j = n;  // 0-based slot of the draw
  c.bonus = n == Lr;
  c.trow = tb + n;
  const float T = a.T[r];
  if (T == 0.0f) {  // p is one-hot at the argmax, and so is the residual
    if (report && lane == 0) {
      a.token[r] = a.row_argmax[c.trow];
      a.is_bonus[r] = c.bonus ? 1 : 0;
    }
    return false;
  }
  c.Td = static_cast<double>(T);
  c.cut = a.row_cut[c.trow];
  c.kept = a.row_kept[c.trow];
  c.trowp = row_ptr(a.tgt, a.dtype, c.trow, a.tgt_ld);
  c.drowp = nullptr;
  c.dlse = 0.0;
  c.nq = 0;
  if (kDense && !c.bonus) {
    c.drowp = row_ptr(a.draft, a.ddtype, static_cast<int64_t>(r) * a.b + n, a.draft_ld);
    c.dlse = a.dlse[pb + n];
  }
  if (!kDense && !c.bonus) {  // branch tokens at slot j with their posterior mass
    if (lane < a.K) {
      c.qtok[lane] = a.branch_tok[(static_cast<size_t>(r) * a.K + lane) * a.b + n];
      c.qw[lane] = a.post_w[(static_cast<size_t>(r) * a.b + n) * a.K + lane];
    }
    c.nq = a.K;
  }
  __syncthreads();  // one wave: orders the LDS table before use
  return true;
}

// p (target, with top-p) and the draw weight w of 8 values of group g
template <bool kDense>
__device__ __forceinline__ void weights8(const SampleArgs& a, const ResCtx& c, int g, bool use_p, double p8[8],
                                         double w8[8]) {
  float l[8];
  load8(c.trowp, a.dtype, g, a.V, l);
#pragma unroll
  for (int k = 0; k < 8; ++k) p8[k] = p_of(l[k], c.cut, c.Td, c.kept);
  if (use_p) {
#pragma unroll
    for (int k = 0; k < 8; ++k) w8[k] = p8[k];
    return;
  }
  if constexpr (kDense) {
    float d[8];
    load8(c.drowp, a.ddtype, g, a.V, d);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double q = exp(static_cast<double>(d[k]) / c.Td - c.dlse);
      const double t = p8[k] - q;
      w8[k] = t > 0.0 ? t : 0.0;
    }
  } else {
    const int v0 = g * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) w8[k] = p8[k];
    for (int t = 0; t < c.nq; ++t) {  // q(v | x_<j) = sum of the posterior over branches at v
      const int dv = c.qtok[t] - v0;
      if (dv >= 0 && dv < 8) {
        double q = 0.0;
        for (int t2 = 0; t2 < c.nq; ++t2)
          if (c.qtok[t2] == c.qtok[t]) q += c.qw[t2];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k == dv) {
            const double d = p8[k] - q;
            w8[k] = d > 0.0 ? d : 0.0;
          }
      }
    }
  }
}

template <bool kDense>
__global__ __launch_bounds__(kWave) void k_res_sums(SampleArgs a) {
  __shared__ ResCtx c;
  const int lane = threadIdx.x;
  const int r = blockIdx.x / a.S;
  const int ch = blockIdx.x % a.S;
  if (!res_setup<kDense>(a, r, false, c)) return;
  const int NG = (a.V + 7) / 8;
  const int g0 = ch * a.CG;
  const int g1 = min(NG, g0 + a.CG);
  double sp = 0.0, sw = 0.0;
  for (int g = g0 + lane; g < g1; g += kWave) {
    double p8[8], w8[8];
    weights8<kDense>(a, c, g, c.bonus, p8, w8);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sp += p8[k];
      sw += w8[k];
    }
  }
  sp = wave_sum_f64(sp);
  sw = wave_sum_f64(sw);
  if (lane == 0) {
    double* pp = a.part + (static_cast<size_t>(r) * a.S + ch) * 2;
    pp[0] = sw;
    pp[1] = sp;
  }
}

template <bool kDense>
__global__ __launch_bounds__(kWave) void k_res_pick(SampleArgs a) {
  __shared__ ResCtx c;
  const int lane = threadIdx.x;
  const int r = blockIdx.x;
  if (!res_setup<kDense>(a, r, true, c)) return;
  const double u = u24(philox_at(*a.seed, static_cast<uint32_t>(c.j), static_cast<uint32_t>(r)).y);
  // chunk sums, one per lane, in chunk order
  const double* pp = a.part + static_cast<size_t>(r) * a.S * 2;
  const double cw = lane < a.S ? pp[lane * 2] : 0.0;
  const bool use_p = c.bonus || !(wave_sum_f64(cw) > 0.0);  // an all-zero residual (rounding) falls back to p
  const double wc = lane < a.S ? pp[lane * 2 + (use_p ? 1 : 0)] : 0.0;
  const double incl = wave_incl_scan_f64(wc);
  const double W = __shfl(incl, kWave - 1, kWave);
  const double t = u * W;
  const uint64_t over = __ballot(lane < a.S && incl > t);
  const int cstar = over ? __ffsll(static_cast<long long>(over)) - 1 : a.S - 1;
  double run = __shfl(incl - wc, cstar, kWave);  // weight before chunk cstar
  // scan chunk cstar, 64 groups (512 values) at a time
  const int NG = (a.V + 7) / 8;
  const int h0 = cstar * a.CG;
  const int h1 = min(NG, h0 + a.CG);
  int found = -1, lastpos = -1;
  for (int gb = h0; gb < h1; gb += kWave) {
    const int g = gb + lane;
    double p8[8], w8[8];
    double loc = 0.0;
    if (g < h1) {
      weights8<kDense>(a, c, g, use_p, p8, w8);
#pragma unroll
      for (int k = 0; k < 8; ++k) loc += w8[k];
    }
    const double inc = wave_incl_scan_f64(loc);
    int mine = -1;
    if (g < h1) {
      double acc = run + (inc - loc);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (w8[k] > 0.0) lastpos = g * 8 + k;
        acc += w8[k];
        if (acc > t && mine < 0) mine = g * 8 + k;
      }
    }
    const uint64_t hit = __ballot(mine >= 0);
    if (hit) {
      found = __shfl(mine, __ffsll(static_cast<long long>(hit)) - 1, kWave);
      break;
    }
    run += __shfl(inc, kWave - 1, kWave);
  }
  if (found < 0) {  // rounding: the last positive weight of the chunk
    int lp = lastpos;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const int q = __shfl_xor(lp, o, kWave);
      lp = q > lp ? q : lp;
    }
    found = lp < 0 ? 0 : lp;
  }
  if (lane == 0) {
    a.token[r] = found;
    a.is_bonus[r] = c.bonus ? 1 : 0;
  }
}

}  // namespace sv

using namespace sv;

static bool sample_args_ok(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V, const int32_t* tgt_off,
                           const int32_t* pos_off, int32_t R, int32_t b, const float* temperature,
                           const int32_t* row_argmax, const float* row_cut, const double* row_kept_lse, int32_t q_mode,
                           const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                           const int32_t* draft_argmax, const double* draft_lse, const uint64_t* seed, void* ws) {
  if (!tgt_logits || !tgt_off || !pos_off || !temperature || !row_argmax || !row_cut || !row_kept_lse || !seed || !ws)
    return false;
  if (R < 1 || b < 1 || b > 64 || V < 1 || tgt_ld < V) return false;
  if (dtype != SV_F32 && dtype != SV_BF16) return false;
  if (!rows_aligned(tgt_logits, dtype, tgt_ld)) return false;
  if (q_mode == SV_Q_DENSE) {
    if (!draft_logits || !draft_argmax || !draft_lse || draft_ld < V) return false;
    if (draft_dtype != SV_F32 && draft_dtype != SV_BF16) return false;
    if (!rows_aligned(draft_logits, draft_dtype, draft_ld)) return false;
  } else if (q_mode != SV_Q_MIXTURE) {
    return false;
  }
  return true;
}

extern "C" int32_t sv_accept(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V, const int32_t* tgt_off,
                             const int32_t* pos_off, int32_t R, int32_t b, const float* temperature,
                             const int32_t* row_argmax, const float* row_cut, const double* row_kept_lse,
                             const int32_t* draft_tok, int32_t q_mode, const void* draft_logits, int32_t draft_dtype,
                             int64_t draft_ld, const int32_t* draft_argmax, const double* draft_lse,
                             const double* q_at_draft, const uint64_t* seed, int32_t* n_acc, double* p_out,
                             double* q_out, float* u_out, void* ws, size_t ws_bytes, void* stream) {
  if (!sample_args_ok(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                      row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed, ws))
    return SV_ERR_ARG;
  if (!draft_tok || !n_acc || (q_mode == SV_Q_MIXTURE && !q_at_draft)) return SV_ERR_ARG;
  if (ws_bytes < 256) return SV_ERR_WORKSPACE;
  SampleArgs a{};
  a.tgt = tgt_logits; a.dtype = dtype; a.tgt_ld = tgt_ld; a.V = V; a.tgt_off = tgt_off; a.pos_off = pos_off;
  a.R = R; a.b = b; a.T = temperature; a.row_argmax = row_argmax; a.row_cut = row_cut; a.row_kept = row_kept_lse;
  a.x = draft_tok; a.q_mode = q_mode; a.draft = draft_logits; a.ddtype = draft_dtype; a.draft_ld = draft_ld;
  a.dargmax = draft_argmax; a.dlse = draft_lse; a.qx = q_at_draft; a.seed = seed; a.n_acc = n_acc;
  a.p_out = p_out; a.q_out = q_out; a.u_out = u_out; a.status = status_word(ws);
  hipLaunchKernelGGL(k_accept, dim3(R), dim3(kWave), 0, static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_residual_sample(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                      const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                                      const float* temperature, const int32_t* row_argmax, const float* row_cut,
                                      const double* row_kept_lse, int32_t q_mode, const void* draft_logits,
                                      int32_t draft_dtype, int64_t draft_ld, const int32_t* draft_argmax,
                                      const double* draft_lse, int32_t K, const int32_t* branch_tok,
                                      const double* post_w, const uint64_t* seed, const int32_t* n_acc,
                                      int32_t* token, int32_t* is_bonus, void* ws, size_t ws_bytes, void* stream) {
  if (!sample_args_ok(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                      row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed, ws))
    return SV_ERR_ARG;
  if (!n_acc || !token || !is_bonus) return SV_ERR_ARG;
  if (q_mode == SV_Q_MIXTURE && (K < 1 || K > 64 || !branch_tok || !post_w)) return SV_ERR_ARG;
  const WsLayout l = ws_layout(R, b, q_mode == SV_Q_MIXTURE ? K : 0, V);
  if (ws_bytes < l.total) return SV_ERR_WORKSPACE;
  const int NG = (V + 7) / 8;
  const int S = res_chunks(V);
  const int CG = (NG + S - 1) / S;
  SampleArgs a{};
  a.tgt = tgt_logits; a.dtype = dtype; a.tgt_ld = tgt_ld; a.V = V; a.tgt_off = tgt_off; a.pos_off = pos_off;
  a.R = R; a.b = b; a.T = temperature; a.row_argmax = row_argmax; a.row_cut = row_cut; a.row_kept = row_kept_lse;
  a.q_mode = q_mode; a.draft = draft_logits; a.ddtype = draft_dtype; a.draft_ld = draft_ld; a.dargmax = draft_argmax;
  a.dlse = draft_lse; a.K = K; a.branch_tok = branch_tok; a.post_w = post_w; a.seed = seed; a.n_acc_in = n_acc;
  a.token = token; a.is_bonus = is_bonus; a.status = status_word(ws);
  a.part = reinterpret_cast<double*>(static_cast<char*>(ws) + l.res_part);
  a.S = S;
  a.CG = CG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_mode == SV_Q_DENSE) {
    hipLaunchKernelGGL(k_res_sums<true>, dim3(R * S), dim3(kWave), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    hipLaunchKernelGGL(k_res_pick<true>, dim3(R), dim3(kWave), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_res_sums<false>, dim3(R * S), dim3(kWave), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    hipLaunchKernelGGL(k_res_pick<false>, dim3(R), dim3(kWave), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
