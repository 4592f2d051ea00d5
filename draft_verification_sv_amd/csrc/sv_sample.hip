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
// Acceptance: one wave per request, one lane per position (b <= 64); p and q at
// the draft token are formed in double; a ballot over the rejecting lanes gives
// the first rejection.
//
// Draw: the sampled row is cut into S <= 64 chunks of up to 1024 8-value groups.
// Chunk sums: one 256-thread block per chunk loads its groups at once and adds
// their weights in double.  With a top-p cut,
// tokens below the cut have weight 0, so each wave first compacts the values
// at or above the cut into LDS and evaluates exp only for those.  Pick (after a
// kernel boundary): one block per request; its first wave scans the chunk sums
// (one per lane) to find the chunk holding u * W, then the block walks that
// chunk 8192 values at a time: per-thread sums of 32 consecutive weights, an
// LDS-staged exclusive block scan, and a block minimum over the first index
// whose running weight exceeds u * W.
//
// The fused tail (sv_accept_sample) runs the category posterior, the
// acceptance tests and the chunk sums in one grid: every chunk block
// recomputes its request's posterior and acceptance (at most 64 positions, a
// few KB of gathers) so that no block waits for another.
#include <math.h>

#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

constexpr int kSumNT = 256;  // threads of a chunk-sum block

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
  const int32_t* branch_tok;
  double* post_w;      // read by the draw; written by the fused tail
  double* q_at_draft;  // written by the fused tail
  const uint64_t* seed;
  const int32_t* n_acc_in;
  int32_t* n_acc;
  int32_t* token;
  int32_t* is_bonus;
  double* p_out;
  double* q_out;
  float* u_out;
  double* part;  // [R * S * 2] chunk sums
  int S;         // chunks per row
  int CG;        // 8-value groups per chunk
  uint32_t* status;
};

__device__ __forceinline__ const char* row_ptr(const void* base, int dtype, int64_t row, int64_t ld) {
  return static_cast<const char*>(base) + static_cast<size_t>(row) * static_cast<size_t>(ld) * (dtype == SV_BF16 ? 2 : 4);
}

// target probability of a token with logit l: [l >= cut] exp(l / T - kept_lse), T > 0
__device__ __forceinline__ double p_of(float l, float cut, double invT, double kept) {
  return l >= cut ? exp(static_cast<double>(l) * invT - kept) : 0.0;
}

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

// Offsets of request r are an exclusive scan with L_r <= b and L_r + 1 target rows.
__device__ __forceinline__ bool request_ok(const SampleArgs& a, int r, int& pb, int& Lr, int& tb) {
  pb = a.pos_off[r];
  Lr = a.pos_off[r + 1] - pb;
  tb = a.tgt_off[r];
  return Lr >= 0 && Lr <= a.b && a.tgt_off[r + 1] - tb == Lr + 1;
}

// ------------------------------------------------------------------ posterior (one wave)
// Lane z < K: f_z = the first position where branch z disagrees with the draft
// (L_r if none).  Branch z is consistent with x_<i iff f_z >= i, and then
// matches x_i iff f_z > i, so
//   w_z^(i) = q(z|y) [f_z >= i] / sum_z' q(z'|y) [f_z' >= i],
//   q(x_i | x_<i) = sum_z w_z^(i) [f_z > i].
// The request's branch tokens and draft tokens, staged in LDS by the whole block
// (one load per thread) so that the recursion below reads no global memory.
struct ReqTables {
  int g[64 * 64];  // [z][i], z < K, i < L_r
  int x[64];
};

__device__ __forceinline__ void stage_tables(const SampleArgs& a, int r, int Lr, ReqTables& t) {
  for (int k = threadIdx.x; k < a.K * Lr; k += blockDim.x) {
    const int z = k / Lr, i = k % Lr;
    t.g[z * 64 + i] = a.branch_tok[(static_cast<size_t>(r) * a.K + z) * a.b + i];
  }
  for (int k = threadIdx.x; k < Lr; k += blockDim.x) t.x[k] = a.x[static_cast<size_t>(r) * a.b + k];
}

__device__ __forceinline__ void branch_agreement(const SampleArgs& a, int r, int Lr, const ReqTables& t, double& pi,
                                                 int& f) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool act = lane < a.K;
  const float ml = act ? a.mix[static_cast<size_t>(r) * a.K + lane] : -INFINITY;
  f = Lr;
  if (act)
    for (int i = Lr - 1; i >= 0; --i)
      if (t.g[lane * 64 + i] != t.x[i]) f = i;
  float mmax = ml;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, o, kWave));
  const double e = act ? exp(static_cast<double>(ml) - static_cast<double>(mmax)) : 0.0;
  pi = e / wave_sum_f64(e);  // q(z | y)
}

// Fills qx[i] for i < L_r; with write_out also post_w, q_at_draft and the status.
__device__ __forceinline__ void posterior_wave(const SampleArgs& a, int r, int Lr, const ReqTables& t, bool write_out,
                                               double* qx, double& pi, int& f) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool act = lane < a.K;
  branch_agreement(a, r, Lr, t, pi, f);
  for (int i = 0; i < Lr; ++i) {
    const double w = act && f >= i ? pi : 0.0;
    const double sw = wave_sum_f64(w);
    const double post = sw > 0.0 ? w / sw : 0.0;
    const double q = wave_sum_f64(f > i ? post : 0.0);
    if (lane == 0) {
      qx[i] = q;
      if (write_out) {
        a.q_at_draft[static_cast<size_t>(r) * a.b + i] = q;
        if (!(sw > 0.0)) raise_status(a.status, SV_ST_EMPTY_POSTERIOR);
      }
    }
    if (write_out && act) a.post_w[(static_cast<size_t>(r) * a.b + i) * a.K + lane] = post;
  }
}

// ------------------------------------------------------------------ acceptance (one wave)
// Lane i < L_r tests position i + 1 (1-based).  q comes from qx (mixture) or
// from the dense draft row.  Returns n_acc on every lane.
__device__ __forceinline__ int accept_wave(const SampleArgs& a, int r, int pb, int Lr, int tb, const double* qx,
                                           bool report) {
  const int i = threadIdx.x & (kWave - 1);
  const uint64_t seed = *a.seed;
  const float T = a.T[r];
  const double invT = 1.0 / static_cast<double>(T);
  bool reject = false;
  if (i < Lr) {
    const int xv = a.x[static_cast<size_t>(r) * a.b + i];
    const bool tok_ok = xv >= 0 && xv < a.V;
    if (report && !tok_ok) raise_status(a.status, SV_ST_BAD_TOKEN);
    const int trow = tb + i;
    double p = 0.0, q = 0.0;
    if (tok_ok) {
      if (T == 0.0f) {
        p = xv == a.row_argmax[trow] ? 1.0 : 0.0;
      } else {
        const float l = load_val_rt(row_ptr(a.tgt, a.dtype, trow, a.tgt_ld), a.dtype, xv);
        p = p_of(l, a.row_cut[trow], invT, a.row_kept[trow]);
      }
      if (a.q_mode == SV_Q_MIXTURE) {
        q = qx[i];
      } else {
        const int pos = pb + i;
        if (T == 0.0f) {
          q = xv == a.dargmax[pos] ? 1.0 : 0.0;
        } else {
          const float d = load_val_rt(row_ptr(a.draft, a.ddtype, static_cast<int64_t>(r) * a.b + i, a.draft_ld),
                                      a.ddtype, xv);
          q = exp(static_cast<double>(d) * invT - a.dlse[pos]);
        }
      }
    }
    const double u = u24(philox_at(seed, static_cast<uint32_t>(i), static_cast<uint32_t>(r)).x);
    const bool accept = q > 0.0 ? (u < p / q) : (p > 0.0);
    reject = !accept;
    if (report) {
      const size_t k = static_cast<size_t>(r) * a.b + i;
      if (a.p_out) a.p_out[k] = p;
      if (a.q_out) a.q_out[k] = q;
      if (a.u_out) a.u_out[k] = static_cast<float>(u);
    }
  }
  const uint64_t mask = __ballot(reject);
  return mask ? (__ffsll(static_cast<long long>(mask)) - 1) : Lr;
}

__global__ __launch_bounds__(kWave) void k_accept(SampleArgs a) {
  const int r = blockIdx.x;
  int pb, Lr, tb;
  if (!request_ok(a, r, pb, Lr, tb)) {
    if (threadIdx.x == 0) {
      raise_status(a.status, SV_ST_BAD_OFFSETS);
      a.n_acc[r] = 0;
    }
    return;
  }
  const double* qx = a.q_mode == SV_Q_MIXTURE ? a.qx + static_cast<size_t>(r) * a.b : nullptr;
  const int n = accept_wave(a, r, pb, Lr, tb, qx, true);
  if (threadIdx.x == 0) a.n_acc[r] = n;
}

// ------------------------------------------------------------------ the draw
// What one request's draw needs.
struct DrawCtx {
  int j, trow;
  bool bonus;
  double invT, kept, dlse;
  float cut;
  const char* trowp;
  const char* drowp;
  int nq;  // mixture: branch entries at slot j with their posterior mass
  int qtok[64];
  double qw[64];
};

// Scalars of the draw context of request r at slot j (thread 0 of the block).
template <bool kDense>
__device__ __forceinline__ void draw_scalars(const SampleArgs& a, int r, int pb, int Lr, int tb, int j, DrawCtx& c) {
  c.j = j;
  c.bonus = j == Lr;
  c.trow = tb + j;
  c.invT = 1.0 / static_cast<double>(a.T[r]);
  c.cut = a.row_cut[tb + j];
  c.kept = a.row_kept[tb + j];
  c.trowp = row_ptr(a.tgt, a.dtype, tb + j, a.tgt_ld);
  c.drowp = nullptr;
  c.dlse = 0.0;
  c.nq = 0;
  if (kDense && j < Lr) {
    c.drowp = row_ptr(a.draft, a.ddtype, static_cast<int64_t>(r) * a.b + j, a.draft_ld);
    c.dlse = a.dlse[pb + j];
  }
  if (!kDense && j < Lr) c.nq = a.K;
}

// q(v | x_<j) of the mixture at token v: the posterior mass of the branches at v
__device__ __forceinline__ double mix_q(const DrawCtx& c, int v) {
  double q = 0.0;
  for (int t = 0; t < c.nq; ++t)
    if (c.qtok[t] == v) q += c.qw[t];
  return q;
}

// p and the draw weight of the 8 values of group g, in vocabulary order
template <bool kDense>
__device__ __forceinline__ void weights8(const SampleArgs& a, const DrawCtx& c, int g, bool use_p, double p8[8],
                                         double w8[8]) {
  float l[8];
  load8(c.trowp, a.dtype, g, a.V, l);
#pragma unroll
  for (int k = 0; k < 8; ++k) p8[k] = p_of(l[k], c.cut, c.invT, c.kept);
  if (use_p || c.bonus) {
#pragma unroll
    for (int k = 0; k < 8; ++k) w8[k] = p8[k];
    return;
  }
  if constexpr (kDense) {
    float d[8];
    load8(c.drowp, a.ddtype, g, a.V, d);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const double q = exp(static_cast<double>(d[k]) * c.invT - c.dlse);
      const double t = p8[k] - q;
      w8[k] = t > 0.0 ? t : 0.0;
    }
  } else {
    const int v0 = g * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) w8[k] = p8[k];
    for (int t = 0; t < c.nq; ++t) {
      const int dv = c.qtok[t] - v0;
      if (dv >= 0 && dv < 8) {
        const double q = mix_q(c, c.qtok[t]);
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

struct SumShared {
  double red[kSumNT / kWave];
  float st[kSumNT / kWave][512];  // per-wave staging of the values at or above the cut
  float sd[kSumNT / kWave][512];  // the matching draft values (dense residual)
};

// Chunk ch of the draw row: sum of p and of the draw weight, in double, to part.
// Each thread prefetches its (up to) 4 groups of a 1024-group super-tile before
// any arithmetic.  The mixture's sparse corrections (branch tokens) are added
// by thread 0.
template <bool kDense>
__device__ void chunk_sums(const SampleArgs& a, const DrawCtx& c, int r, int ch, SumShared& sh) {
  constexpr int TILES = 4;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wv = tid / kWave;
  const int NG = (a.V + 7) / 8;
  const int g0 = ch * a.CG;
  const int g1 = min(NG, g0 + a.CG);
  const bool dense_res = kDense && !c.bonus;
  const bool cut_on = c.cut > -INFINITY;
  double sp = 0.0, sw = 0.0;
  for (int sb = g0; sb < g1; sb += TILES * kSumNT) {
    float l[TILES][8], d[TILES][8];
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
      const int g = sb + k * kSumNT + tid;
      if (g < g1) {
        load8(c.trowp, a.dtype, g, a.V, l[k]);
        if (dense_res) load8(c.drowp, a.ddtype, g, a.V, d[k]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) l[k][q] = -INFINITY;
      }
    }
    if (!cut_on) {
#pragma unroll
      for (int k = 0; k < TILES; ++k) {
        if (sb + k * kSumNT + tid >= g1) continue;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const double p = exp(static_cast<double>(l[k][q]) * c.invT - c.kept);
          sp += p;
          if (dense_res) {
            const double t = p - exp(static_cast<double>(d[k][q]) * c.invT - c.dlse);
            sw += t > 0.0 ? t : 0.0;
          } else {
            sw += p;
          }
        }
      }
    } else {
      // top-p: only values at or above the cut carry weight; compact them per wave
#pragma unroll
      for (int k = 0; k < TILES; ++k) {
        uint32_t m = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q) m |= (l[k][q] >= c.cut ? 1u : 0u) << q;
        const int cnt = __popc(m);
        const int inc = wave_incl_scan_i32(cnt);
        const int tot = __shfl(inc, kWave - 1, kWave);
        int o = inc - cnt;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (m & (1u << q)) {
            sh.st[wv][o] = l[k][q];
            if (dense_res) sh.sd[wv][o] = d[k][q];
            ++o;
          }
        __syncthreads();
        for (int e = lane; e < tot; e += kWave) {
          const double p = exp(static_cast<double>(sh.st[wv][e]) * c.invT - c.kept);
          sp += p;
          if (dense_res) {
            const double t = p - exp(static_cast<double>(sh.sd[wv][e]) * c.invT - c.dlse);
            sw += t > 0.0 ? t : 0.0;
          } else {
            sw += p;
          }
        }
        __syncthreads();
      }
    }
  }
  sp = block_sum_f64<kSumNT>(sp, sh.red);
  sw = block_sum_f64<kSumNT>(sw, sh.red);
  if (tid == 0) {
    if (!kDense && !c.bonus) {  // branch tokens: weight max(0, p - q) instead of p
      const int v0 = g0 * 8, v1 = min(a.V, g1 * 8);
      for (int t = 0; t < c.nq; ++t) {
        const int v = c.qtok[t];
        bool first = true;
        for (int t2 = 0; t2 < t; ++t2)
          if (c.qtok[t2] == v) first = false;
        if (!first || v < v0 || v >= v1) continue;
        const double p = p_of(load_val_rt(c.trowp, a.dtype, v), c.cut, c.invT, c.kept);
        const double dq = p - mix_q(c, v);
        sw += (dq > 0.0 ? dq : 0.0) - p;
      }
    }
    double* pp = a.part + (static_cast<size_t>(r) * a.S + ch) * 2;
    pp[0] = sw;
    pp[1] = sp;
  }
}

struct TailShared {
  DrawCtx c;
  SumShared s;
  ReqTables t;
  double qx[64];
  int n;
};

// Standalone chunk sums (sv_residual_sample): n_acc is an input.
template <bool kDense>
__global__ __launch_bounds__(kSumNT) void k_res_sums(SampleArgs a) {
  __shared__ TailShared sh;
  const int r = blockIdx.x / a.S, ch = blockIdx.x % a.S;
  const int tid = threadIdx.x;
  int pb, Lr, tb;
  if (!request_ok(a, r, pb, Lr, tb)) return;
  if (a.T[r] == 0.0f) return;  // the draw is the argmax
  int n = a.n_acc_in[r];
  n = n < 0 ? 0 : (n > Lr ? Lr : n);
  if (tid == 0) draw_scalars<kDense>(a, r, pb, Lr, tb, n, sh.c);
  if (!kDense && n < Lr && tid < a.K) {
    sh.c.qtok[tid] = a.branch_tok[(static_cast<size_t>(r) * a.K + tid) * a.b + n];
    sh.c.qw[tid] = a.post_w[(static_cast<size_t>(r) * a.b + n) * a.K + tid];
  }
  __syncthreads();
  chunk_sums<kDense>(a, sh.c, r, ch, sh.s);
}

// Fused tail: posterior (mixture), acceptance, then the chunk sums of the draw.
template <bool kDense>
__global__ __launch_bounds__(kSumNT) void k_tail_sums(SampleArgs a) {
  __shared__ TailShared sh;
  const int r = blockIdx.x / a.S, ch = blockIdx.x % a.S;
  const int tid = threadIdx.x;
  int pb, Lr, tb;
  if (!request_ok(a, r, pb, Lr, tb)) {
    if (ch == 0 && tid == 0) {
      raise_status(a.status, SV_ST_BAD_OFFSETS);
      a.n_acc[r] = 0;
    }
    return;
  }
  const bool report = ch == 0;
  if (!kDense) {
    stage_tables(a, r, Lr, sh.t);
    __syncthreads();
  }
  if (tid < kWave) {
    double pi = 0.0;
    int f = 0;
    if (!kDense) posterior_wave(a, r, Lr, sh.t, report, sh.qx, pi, f);
    const int n = accept_wave(a, r, pb, Lr, tb, sh.qx, report);
    if (tid == 0) {
      sh.n = n;
      if (report) a.n_acc[r] = n;
      if (a.T[r] != 0.0f) draw_scalars<kDense>(a, r, pb, Lr, tb, n, sh.c);
    }
    if (!kDense && n < Lr) {
      // branch tokens and posterior mass at the draw slot (as posterior_wave formed them)
      const bool act = tid < a.K;
      const double w = act && f >= n ? pi : 0.0;
      const double sw = wave_sum_f64(w);
      if (act) {
        sh.c.qw[tid] = sw > 0.0 ? w / sw : 0.0;
        sh.c.qtok[tid] = sh.t.g[tid * 64 + n];
      }
    }
  }
  __syncthreads();
  if (a.T[r] == 0.0f) return;  // the draw is the argmax (taken by the pick kernel)
  chunk_sums<kDense>(a, sh.c, r, ch, sh.s);
}

// The draw: one 256-thread block per request, after the chunk sums.
template <bool kDense>
__global__ __launch_bounds__(kSumNT) void k_res_pick(SampleArgs a) {
  __shared__ DrawCtx c;
  __shared__ double red[kSumNT / kWave];
  __shared__ int redi[kSumNT / kWave];
  __shared__ int s_cstar, s_use_p;
  __shared__ double s_base, s_t;
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  int pb, Lr, tb;
  if (!request_ok(a, r, pb, Lr, tb)) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  int n = a.n_acc_in[r];
  if (n < 0 || n > Lr) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_NACC);
    n = n < 0 ? 0 : Lr;
  }
  if (a.T[r] == 0.0f) {  // p is one-hot at the argmax, and so is the residual
    if (tid == 0) {
      a.token[r] = a.row_argmax[tb + n];
      a.is_bonus[r] = n == Lr ? 1 : 0;
    }
    return;
  }
  if (tid == 0) draw_scalars<kDense>(a, r, pb, Lr, tb, n, c);
  if (!kDense && n < Lr && tid < a.K) {
    c.qtok[tid] = a.branch_tok[(static_cast<size_t>(r) * a.K + tid) * a.b + n];
    c.qw[tid] = a.post_w[(static_cast<size_t>(r) * a.b + n) * a.K + tid];
  }
  if (tid < kWave) {  // wave 0: the chunk holding u * W, from the chunk sums (one per lane)
    const int lane = tid;
    const double u = u24(philox_at(*a.seed, static_cast<uint32_t>(n), static_cast<uint32_t>(r)).y);
    const double* pp = a.part + static_cast<size_t>(r) * a.S * 2;
    const double cw = lane < a.S ? pp[lane * 2] : 0.0;
    const bool use_p = n == Lr || !(wave_sum_f64(cw) > 0.0);  // an all-zero residual (rounding) falls back to p
    const double wc = lane < a.S ? pp[lane * 2 + (use_p ? 1 : 0)] : 0.0;
    const double incl = wave_incl_scan_f64(wc);
    const double W = __shfl(incl, kWave - 1, kWave);
    const double t = u * W;
    const uint64_t over = __ballot(lane < a.S && incl > t);
    const int cstar = over ? __ffsll(static_cast<long long>(over)) - 1 : a.S - 1;
    const double base = __shfl(incl - wc, cstar, kWave);  // weight before chunk cstar
    if (lane == 0) {
      s_cstar = cstar;
      s_use_p = use_p ? 1 : 0;
      s_base = base;
      s_t = t;
    }
  }
  __syncthreads();
  const bool use_p = s_use_p != 0;
  const double t = s_t;
  // walk chunk cstar: thread tid takes GPT consecutive groups (loaded at once),
  // an exclusive block scan of the per-thread sums finds the thread holding t
  constexpr int GPT = 4;
  const int NG = (a.V + 7) / 8;
  const int h0 = s_cstar * a.CG;
  const int h1 = min(NG, h0 + a.CG);
  double run = s_base;
  int found = 0x7FFFFFFF, lastpos = -1;
  for (int sb = h0; sb < h1; sb += GPT * kSumNT) {
    const int gs = sb + tid * GPT;
    double w[GPT][8];
    double loc = 0.0;
#pragma unroll
    for (int k = 0; k < GPT; ++k) {
      double p8[8];
      if (gs + k < h1) {
        weights8<kDense>(a, c, gs + k, use_p, p8, w[k]);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) w[k][q] = 0.0;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) loc += w[k][q];
    }
    double tile;
    const double excl = block_excl_scan_f64<kSumNT>(loc, red, &tile);
    double acc = run + excl;
#pragma unroll
    for (int k = 0; k < GPT; ++k)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (w[k][q] > 0.0) lastpos = (gs + k) * 8 + q;
        acc += w[k][q];
        if (acc > t && found == 0x7FFFFFFF) found = (gs + k) * 8 + q;
      }
    const int fmin = block_min_i32<kSumNT>(found, redi);
    if (fmin != 0x7FFFFFFF) {
      found = fmin;
      break;
    }
    run += tile;
  }
  if (found == 0x7FFFFFFF) {  // rounding: the last positive weight of the chunk
    found = -block_min_i32<kSumNT>(-lastpos, redi);
    if (found < 0) found = 0;
  }
  if (tid == 0) {
    a.token[r] = found;
    a.is_bonus[r] = n == Lr ? 1 : 0;
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

static SampleArgs sample_args(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V, const int32_t* tgt_off,
                              const int32_t* pos_off, int32_t R, int32_t b, const float* temperature,
                              const int32_t* row_argmax, const float* row_cut, const double* row_kept_lse,
                              int32_t q_mode, const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                              const int32_t* draft_argmax, const double* draft_lse, const uint64_t* seed, void* ws) {
  SampleArgs a{};
  a.tgt = tgt_logits; a.dtype = dtype; a.tgt_ld = tgt_ld; a.V = V; a.tgt_off = tgt_off; a.pos_off = pos_off;
  a.R = R; a.b = b; a.T = temperature; a.row_argmax = row_argmax; a.row_cut = row_cut; a.row_kept = row_kept_lse;
  a.q_mode = q_mode; a.draft = draft_logits; a.ddtype = draft_dtype; a.draft_ld = draft_ld;
  a.dargmax = draft_argmax; a.dlse = draft_lse; a.seed = seed; a.status = status_word(ws);
  const WsLayout l = ws_layout(R, b, 0, V);
  a.part = reinterpret_cast<double*>(static_cast<char*>(ws) + l.res_part);
  a.S = res_chunks(V);
  a.CG = ((V + 7) / 8 + a.S - 1) / a.S;
  return a;
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
  SampleArgs a = sample_args(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                             row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed,
                             ws);
  a.x = draft_tok; a.qx = q_at_draft; a.n_acc = n_acc; a.p_out = p_out; a.q_out = q_out; a.u_out = u_out;
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
  if (ws_bytes < ws_layout(R, b, q_mode == SV_Q_MIXTURE ? K : 0, V).total) return SV_ERR_WORKSPACE;
  SampleArgs a = sample_args(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                             row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed,
                             ws);
  a.K = q_mode == SV_Q_MIXTURE ? K : 0; a.branch_tok = branch_tok; a.post_w = const_cast<double*>(post_w);
  a.n_acc_in = n_acc; a.token = token; a.is_bonus = is_bonus;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_mode == SV_Q_DENSE) {
    hipLaunchKernelGGL(k_res_sums<true>, dim3(R * a.S), dim3(kSumNT), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    hipLaunchKernelGGL(k_res_pick<true>, dim3(R), dim3(kSumNT), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_res_sums<false>, dim3(R * a.S), dim3(kSumNT), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    hipLaunchKernelGGL(k_res_pick<false>, dim3(R), dim3(kSumNT), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_accept_sample(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                    const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                                    const float* temperature, const int32_t* row_argmax, const float* row_cut,
                                    const double* row_kept_lse, const int32_t* draft_tok, int32_t q_mode,
                                    const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                                    const int32_t* draft_argmax, const double* draft_lse, int32_t K,
                                    const float* mix_logits, const int32_t* branch_tok, double* post_w,
                                    double* q_at_draft, const uint64_t* seed, int32_t* n_acc, int32_t* token,
                                    int32_t* is_bonus, double* p_out, double* q_out, float* u_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!sample_args_ok(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                      row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed, ws))
    return SV_ERR_ARG;
  if (!draft_tok || !n_acc || !token || !is_bonus) return SV_ERR_ARG;
  if (q_mode == SV_Q_MIXTURE && (K < 1 || K > 64 || !mix_logits || !branch_tok || !post_w || !q_at_draft))
    return SV_ERR_ARG;
  if (ws_bytes < ws_layout(R, b, q_mode == SV_Q_MIXTURE ? K : 0, V).total) return SV_ERR_WORKSPACE;
  SampleArgs a = sample_args(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                             row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed,
                             ws);
  a.x = draft_tok; a.K = q_mode == SV_Q_MIXTURE ? K : 0; a.mix = mix_logits; a.branch_tok = branch_tok;
  a.post_w = post_w; a.q_at_draft = q_at_draft; a.n_acc = n_acc; a.n_acc_in = n_acc; a.token = token;
  a.is_bonus = is_bonus; a.p_out = p_out; a.q_out = q_out; a.u_out = u_out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_mode == SV_Q_DENSE) {
    hipLaunchKernelGGL(k_tail_sums<true>, dim3(R * a.S), dim3(kSumNT), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    hipLaunchKernelGGL(k_res_pick<true>, dim3(R), dim3(kSumNT), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_tail_sums<false>, dim3(R * a.S), dim3(kSumNT), 0, s, a);
    if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
    hipLaunchKernelGGL(k_res_pick<false>, dim3(R), dim3(kSumNT), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
