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
// Two launches per step, both built as short chains of independent loads:
//
// Sums (one 256-thread block per (request, chunk of 1024 8-value groups)):
//   A. the request's offsets, temperature, seed, draft tokens, mixing logits
//      and branch tokens, each by its own thread;
//   B. the row statistics of the L_r + 1 candidate rows, the target (and
//      dense draft) logits at the draft tokens, and the target logits at every
//      branch token, each by its own thread;
//   C. one wave: the category posterior in closed form, the acceptance tests,
//      the first rejection n, and the draw context of slot n;
//   D. the chunk of the drawn row: each wave sums p and the draw weight over
//      its 512-value sub-chunks (exp only over the values at or above the
//      top-p cut, packed first) and writes one pair of doubles per sub-chunk.
// Every chunk block recomputes A-C (at most 64 positions, a few KB of
// gathers), so that no block waits for another; the first one writes the
// acceptance outputs and the draw record.
//
// Pick (one wave per request): a wave scan over the request's sub-chunk sums
// finds the sub-chunk holding u * W; the wave then re-forms its 512 weights
// and scans them.
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
  const double* qx;  // q at the draft tokens (mixture, standalone acceptance)
  int K;
  const float* mix;  // mixing logits (fused tail)
  const int32_t* branch_tok;
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

// ------------------------------------------------------------------ standalone acceptance (one wave)
// Lane i < L_r tests position i + 1 (1-based).  q comes from the given
// q_at_draft (mixture) or from the dense draft row.  Returns n_acc on every lane.
__device__ __forceinline__ int accept_wave(const SampleArgs& a, int r, int pb, int Lr, int tb, const double* qx) {
  const int i = threadIdx.x & (kWave - 1);
  const uint64_t seed = *a.seed;
  const float T = a.T[r];
  const double invT = 1.0 / static_cast<double>(T);
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
    const size_t k = static_cast<size_t>(r) * a.b + i;
    if (a.p_out) a.p_out[k] = p;
    if (a.q_out) a.q_out[k] = q;
    if (a.u_out) a.u_out[k] = static_cast<float>(u);
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
  const int n = accept_wave(a, r, pb, Lr, tb, qx);
  if (threadIdx.x == 0) a.n_acc[r] = n;
}

// ------------------------------------------------------------------ the draw
// What the chunk blocks of one request share (built by wave 0).
struct DrawCtx {
  int mode, n, bonus, token, ncorr;
  float cut;
  double invT, kept, dlse;
  int64_t trow, drow;
  int ctok[64];
  double cp[64];  // p at ctok
  double cw[64];  // draw weight at ctok
};

struct TailShared {
  // A. request header and tables
  int pb, pe, tb, te, nin;
  float T;
  uint64_t seed;
  int x[64];
  float mix[64];
  // B. statistics of the candidate rows tb + i (i <= L_r), values at the draft
  // tokens, and f_z (the first position where branch z leaves the draft)
  float rc[65];
  double rk[65];
  int ra[65];
  float lx[64], dx[64];
  double dl[64];
  int da[64];
  int f[64];
  // standalone draw: branch tokens and posterior weights at the slot
  int tv[64];
  double tw[64];
  DrawCtx c;
  // D. per-wave lists of the values at or above the cut (and their draft values)
  float st[kSumNT / kWave][kSubG * 8];
  float sd[kSumNT / kWave][kSubG * 8];
};

// Mixture residual at the draw slot (wave 0): lane z < K holds branch z (whether
// it is consistent with the accepted prefix, its token v, its posterior weight
// w and the target logit at v).  q(v) is the summed weight of the branches with
// token v; the draw weight at v is max(0, p(v) - q(v)); every other token keeps
// p.  The distinct tokens go to c.ctok in lane order.
__device__ __forceinline__ void build_corrections(DrawCtx& c, int K, bool act, int v, double w, float lv) {
  const int lane = threadIdx.x & (kWave - 1);
  const int va = act ? v : -1;
  const double wa = act ? w : 0.0;
  bool first = act;
  double q = 0.0;
  for (int z = 0; z < K; ++z) {
    const int vz = bcast_i32(va, z);
    const double wz = bcast_f64(wa, z);
    if (act && vz == v) {
      q += wz;
      if (z < lane) first = false;
    }
  }
  const uint64_t fm = __ballot(first);
  if (first) {
    const int idx = __popcll(fm & ((1ull << lane) - 1ull));
    const double p = p_of(lv, c.cut, c.invT, c.kept);
    const double d = p - q;
    c.ctok[idx] = v;
    c.cp[idx] = p;
    c.cw[idx] = d > 0.0 ? d : 0.0;
  }
  if (lane == 0) c.ncorr = __popcll(fm);
}

// The first chunk block's copy of the context for the pick kernel (wave 0).
__device__ __forceinline__ void write_record(const SampleArgs& a, int r, const DrawCtx& c) {
  const int lane = threadIdx.x & (kWave - 1);
  DrawRec& d = a.rec[r];
  if (lane == 0) {
    d.mode = c.mode; d.n = c.n; d.bonus = c.bonus; d.token = c.token; d.ncorr = c.ncorr;
    d.trow = c.trow; d.drow = c.drow; d.cut = c.cut; d.invT = c.invT; d.kept = c.kept; d.dlse = c.dlse;
  }
  if (lane < c.ncorr) {
    d.ctok[lane] = c.ctok[lane];
    d.cw[lane] = c.cw[lane];
  }
}

// D. Sums of p and of the draw weight over the sub-chunks of chunk ch of the
// drawn row; wave wv takes sub-chunks ch*16 + k*4 + wv, k < 4, one 8-value
// group per lane, all loaded before any arithmetic.  Only values at or above
// the top-p cut carry weight, so each sub-chunk's such values are first packed
// densely into the wave's LDS list (a ballot per value slot gives each lane its
// position) and exp runs over the packed list only.
template <bool kDense>
__device__ __forceinline__ void sub_sums(const SampleArgs& a, const DrawCtx& c, int r, int ch, float* st, float* sd) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int NG = groups_of(a.V);
  const bool dense_res = kDense && c.mode == kDrawResidual;
  const bool mix_res = !kDense && c.mode == kDrawResidual;
  const char* trowp = row_ptr(a.tgt, a.dtype, c.trow, a.tgt_ld);
  const char* drowp = dense_res ? row_ptr(a.draft, a.ddtype, c.drow, a.draft_ld) : nullptr;
  const int sub0 = ch * kChunkSubs + wv;
  float l[kSubPerWave][8], d[kSubPerWave][8];
#pragma unroll
  for (int k = 0; k < kSubPerWave; ++k) {
    const int g = (sub0 + k * (kSumNT / kWave)) * kSubG + lane;
    if (g < NG) {
      load8(trowp, a.dtype, g, a.V, l[k]);
      if (dense_res) load8(drowp, a.ddtype, g, a.V, d[k]);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) l[k][q] = -INFINITY;
    }
  }
#pragma unroll
  for (int k = 0; k < kSubPerWave; ++k) {
    const int sub = sub0 + k * (kSumNT / kWave);
    if (sub >= a.NSUB) break;  // wave-uniform
    int tot = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const bool keep = l[k][q] >= c.cut;  // -inf padding fails unless the cut is -inf (then it weighs 0)
      const uint64_t m = __ballot(keep);
      if (keep) {
        const int o = tot + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
        st[o] = l[k][q];
        if (dense_res) sd[o] = d[k][q];
      }
      tot += __popcll(m);
    }
    __syncwarp();
    double sp = 0.0, sw = 0.0;
    for (int e = lane; e < tot; e += kWave) {
      const double p = exp(static_cast<double>(st[e]) * c.invT - c.kept);
      sp += p;
      if (dense_res) {
        const double t = p - exp(static_cast<double>(sd[e]) * c.invT - c.dlse);
        sw += t > 0.0 ? t : 0.0;
      }
    }
    __syncwarp();  // the list is rewritten by the next sub-chunk
    sp = wave_sum_f64(sp);
    if (dense_res) sw = wave_sum_f64(sw);
    if (lane == 0) {
      if (!dense_res) sw = sp;
      if (mix_res) {  // branch tokens: weight max(0, p - q) instead of p
        const int v0 = sub * kSubG * 8;
        for (int t = 0; t < c.ncorr; ++t) {
          const int v = c.ctok[t];
          if (v >= v0 && v < v0 + kSubG * 8) sw += c.cw[t] - c.cp[t];
        }
      }
      double* pp = a.sub + (static_cast<size_t>(r) * a.NSUB + sub) * 2;
      pp[0] = sw;
      pp[1] = sp;
    }
  }
}

// The fused tail (kAccept: posterior, acceptance and the draw's sums) or the
// standalone draw's sums (n from n_acc_in, posterior weights from post_w).
template <bool kDense, bool kAccept>
__global__ __launch_bounds__(kSumNT) void k_draw_sums(SampleArgs a) {
  __shared__ TailShared sh;
  extern __shared__ int dyn[];  // mixture: branch tokens [K][b], then target logits at them [K][b]
  int* g = dyn;
  float* gl = reinterpret_cast<float*>(dyn + a.K * a.b);
  const int r = blockIdx.x / a.S, ch = blockIdx.x % a.S;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const bool report = ch == 0;
  const int K = kDense ? 0 : a.K, b = a.b;
  DrawCtx& c = sh.c;

  // A. independent loads
  if (tid == 0) {
    sh.pb = a.pos_off[r];
    sh.pe = a.pos_off[r + 1];
    sh.tb = a.tgt_off[r];
    sh.te = a.tgt_off[r + 1];
    sh.T = a.T[r];
    sh.seed = *a.seed;
    sh.nin = kAccept ? 0 : a.n_acc_in[r];
  }
  if (tid < kWave) sh.f[tid] = 0x7FFFFFFF;
  if (kAccept) {
    for (int i = tid; i < b; i += kSumNT) sh.x[i] = a.x[static_cast<size_t>(r) * b + i];
    if (!kDense) {
      for (int z = tid; z < K; z += kSumNT) sh.mix[z] = a.mix[static_cast<size_t>(r) * K + z];
      for (int k = tid; k < K * b; k += kSumNT) g[k] = a.branch_tok[static_cast<size_t>(r) * K * b + k];
    }
  }
  __syncthreads();
  const int pb = sh.pb, tb = sh.tb, Lr = sh.pe - sh.pb;
  if (!(Lr >= 0 && Lr <= b && sh.te - tb == Lr + 1)) {
    if (report && tid == 0) {
      raise_status(a.status, SV_ST_BAD_OFFSETS);
      if (kAccept) a.n_acc[r] = 0;
      a.rec[r].mode = kDrawNone;
    }
    return;
  }
  const bool greedy = sh.T == 0.0f;
  const double invT = 1.0 / static_cast<double>(sh.T);

  if (kAccept) {
    // B. row statistics of the candidate rows, values at the draft and branch
    // tokens; f_z = the first position where branch z leaves the draft
    for (int i = tid; i <= Lr; i += kSumNT) {
      sh.rc[i] = a.row_cut[tb + i];
      sh.rk[i] = a.row_kept[tb + i];
      sh.ra[i] = a.row_argmax[tb + i];
    }
    for (int i = tid; i < Lr; i += kSumNT) {
      const int xv = sh.x[i];
      const bool ok = xv >= 0 && xv < a.V;
      sh.lx[i] = ok ? load_val_rt(row_ptr(a.tgt, a.dtype, tb + i, a.tgt_ld), a.dtype, xv) : -INFINITY;
      if (kDense) {
        sh.dx[i] = ok ? load_val_rt(row_ptr(a.draft, a.ddtype, static_cast<int64_t>(r) * b + i, a.draft_ld),
                                    a.ddtype, xv)
                      : -INFINITY;
        sh.dl[i] = a.dlse[pb + i];
        sh.da[i] = a.dargmax[pb + i];
      }
    }
    if (!kDense)
      for (int k = tid; k < K * Lr; k += kSumNT) {
        const int z = k / Lr, i = k - z * Lr;
        const int v = g[z * b + i];
        if (v != sh.x[i]) atomicMin(&sh.f[z], i);
        gl[z * b + i] = v >= 0 && v < a.V ? load_val_rt(row_ptr(a.tgt, a.dtype, tb + i, a.tgt_ld), a.dtype, v)
                                          : -INFINITY;
      }
    __syncthreads();

    // C. acceptance, posterior and draw context (wave 0; lane i < L_r tests
    // position i + 1)
    if (tid < kWave) {
      const bool pos = lane < Lr;
      const int xv = pos ? sh.x[lane] : -1;
      const bool ok = xv >= 0 && xv < a.V;
      if (report && pos && !ok) raise_status(a.status, SV_ST_BAD_TOKEN);
      double p = 0.0, q = 0.0;
      if (ok) {
        p = greedy ? (xv == sh.ra[lane] ? 1.0 : 0.0) : p_of(sh.lx[lane], sh.rc[lane], invT, sh.rk[lane]);
        if (kDense)
          q = greedy ? (xv == sh.da[lane] ? 1.0 : 0.0) : exp(static_cast<double>(sh.dx[lane]) * invT - sh.dl[lane]);
      }
      const double u = u24(philox_at(sh.seed, static_cast<uint32_t>(lane), static_cast<uint32_t>(r)).x);
      double pi = 0.0, A = 0.0;  // lane z: pi_z; lane i: A(i)
      int f = -1;
      if (!kDense) {
        // Lane z < K: pi_z = q(z | y), f_z as above (L_r if none).  With
        // A(i) = sum_z pi_z [f_z >= i]: w_z^(i) = pi_z [f_z >= i] / A(i) and
        // q(x_i | x_<i) = A(i + 1) / A(i).
        const bool act = lane < K;
        const float ml = act ? sh.mix[lane] : -INFINITY;
        const float mmax = wave_max_f32(ml);
        const double e = act ? exp(static_cast<double>(ml) - static_cast<double>(mmax)) : 0.0;
        pi = e / wave_sum_f64(e);
        f = act ? min(sh.f[lane], Lr) : -1;
        double Ai = 0.0, Ai1 = 0.0;
        for (int z = 0; z < K; ++z) {
          const double pz = bcast_f64(pi, z);
          const int fz = bcast_i32(f, z);
          Ai += fz >= lane ? pz : 0.0;
          Ai1 += fz > lane ? pz : 0.0;
        }
        if (pos) {
          if (ok) q = Ai > 0.0 ? Ai1 / Ai : 0.0;
          if (report) {
            a.q_at_draft[static_cast<size_t>(r) * b + lane] = Ai > 0.0 ? Ai1 / Ai : 0.0;
            if (!(Ai > 0.0)) raise_status(a.status, SV_ST_EMPTY_POSTERIOR);
          }
        }
        if (report) {  // post_w[i][z], lane i < L_r
          double* pw = a.post_w + static_cast<size_t>(r) * b * K;
          for (int z = 0; z < K; ++z) {
            const double pz = bcast_f64(pi, z);
            const int fz = bcast_i32(f, z);
            if (pos) pw[lane * K + z] = Ai > 0.0 && fz >= lane ? pz / Ai : 0.0;
          }
        }
        A = Ai;
      }
      bool reject = false;
      if (pos) {
        reject = !(q > 0.0 ? u < p / q : p > 0.0);
        if (report) {
          const size_t k = static_cast<size_t>(r) * b + lane;
          if (a.p_out) a.p_out[k] = p;
          if (a.q_out) a.q_out[k] = q;
          if (a.u_out) a.u_out[k] = static_cast<float>(u);
        }
      }
      const uint64_t mask = __ballot(reject);
      const int n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : Lr;
      if (report && lane == 0) a.n_acc[r] = n;
      if (lane == 0) {
        c.n = n;
        c.bonus = n == Lr ? 1 : 0;
        c.mode = greedy ? kDrawGreedy : (n == Lr ? kDrawP : kDrawResidual);
        c.token = sh.ra[n];
        c.cut = sh.rc[n];
        c.kept = sh.rk[n];
        c.invT = invT;
        c.dlse = kDense && n < Lr ? sh.dl[n] : 0.0;
        c.trow = tb + n;
        c.drow = static_cast<int64_t>(r) * b + n;
        c.ncorr = 0;
      }
      __syncwarp();
      if (!kDense && !greedy && n < Lr) {
        const double An = bcast_f64(A, n);
        const bool act = lane < K && f >= n;
        build_corrections(c, K, act, act ? g[lane * b + n] : -1, act ? pi / An : 0.0,
                          act ? gl[lane * b + n] : -INFINITY);
      }
      __syncwarp();
      if (report) write_record(a, r, c);
    }
  } else {
    // standalone draw: n given; branch tokens and posterior weights at slot n given
    int n = sh.nin;
    if (n < 0 || n > Lr) {
      if (report && tid == 0) raise_status(a.status, SV_ST_BAD_NACC);
      n = n < 0 ? 0 : Lr;
    }
    const bool mres = !kDense && !greedy && n < Lr;
    if (tid == 0) {
      c.n = n;
      c.bonus = n == Lr ? 1 : 0;
      c.mode = greedy ? kDrawGreedy : (n == Lr ? kDrawP : kDrawResidual);
      c.token = a.row_argmax[tb + n];
      c.cut = a.row_cut[tb + n];
      c.kept = a.row_kept[tb + n];
      c.invT = invT;
      c.dlse = kDense && n < Lr ? a.dlse[pb + n] : 0.0;
      c.trow = tb + n;
      c.drow = static_cast<int64_t>(r) * b + n;
      c.ncorr = 0;
    }
    if (mres && tid < K) {
      sh.tv[tid] = a.branch_tok[(static_cast<size_t>(r) * K + tid) * b + n];
      sh.tw[tid] = a.post_w[(static_cast<size_t>(r) * b + n) * K + tid];
    }
    __syncthreads();
    if (tid < kWave) {
      if (mres) {
        const bool in = lane < K;
        const int v = in ? sh.tv[lane] : -1;
        const double w = in ? sh.tw[lane] : 0.0;
        const bool act = in && w > 0.0 && v >= 0 && v < a.V;
        const float lv = act ? load_val_rt(row_ptr(a.tgt, a.dtype, tb + n, a.tgt_ld), a.dtype, v) : -INFINITY;
        build_corrections(c, K, act, v, w, lv);
      }
      __syncwarp();
      if (report) write_record(a, r, c);
    }
  }
  __syncthreads();
  if (c.mode == kDrawGreedy) return;  // the draw is the argmax (taken by the pick kernel)
  const int wv = tid / kWave;
  sub_sums<kDense>(a, c, r, ch, sh.st[wv], sh.sd[wv]);
}

// The draw: one wave per request, after the sums.  Lane l holds the sub-chunk
// sums [l*spt, (l+1)*spt); a wave scan finds the sub-chunk holding t = u * W,
// then the lanes take its 64 groups and a second scan finds the token.
constexpr int kPickCache = 8;  // sub-chunk sums kept in registers per lane

template <bool kDense>
__global__ __launch_bounds__(kWave) void k_pick(SampleArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const DrawRec& rec = a.rec[r];
  const int mode = rec.mode, n = rec.n, bonus = rec.bonus;
  const uint64_t seed = *a.seed;
  const int NSUB = a.NSUB;
  const int spt = (NSUB + kWave - 1) / kWave;
  const int s0 = min(NSUB, lane * spt), s1 = min(NSUB, s0 + spt);
  const double* subp = a.sub + static_cast<size_t>(r) * NSUB * 2;
  // every load of this round is independent of the others
  double cw_[kPickCache], cp_[kPickCache];
  double lw = 0.0, lp = 0.0;
#pragma unroll
  for (int k = 0; k < kPickCache; ++k) {
    const int s = s0 + k;
    cw_[k] = s < s1 ? subp[2 * s] : 0.0;
    cp_[k] = s < s1 ? subp[2 * s + 1] : 0.0;
  }
#pragma unroll
  for (int k = 0; k < kPickCache; ++k) {
    lw += cw_[k];
    lp += cp_[k];
  }
  for (int s = s0 + kPickCache; s < s1; ++s) {
    lw += subp[2 * s];
    lp += subp[2 * s + 1];
  }
  const int ctok = kDense ? -1 : rec.ctok[lane];
  const double cwt = kDense ? 0.0 : rec.cw[lane];
  if (mode == kDrawNone) return;  // malformed offsets (reported by the sums kernel)
  if (mode == kDrawGreedy) {      // p is one-hot at the argmax, and so is the residual
    if (lane == 0) {
      a.token[r] = rec.token;
      a.is_bonus[r] = bonus;
    }
    return;
  }
  bool use_p = mode == kDrawP;
  double incl = wave_incl_scan_f64(use_p ? lp : lw);
  double W = bcast_f64(incl, kWave - 1);
  if (!use_p && !(W > 0.0)) {  // an all-zero residual (rounding) falls back to p
    use_p = true;
    incl = wave_incl_scan_f64(lp);
    W = bcast_f64(incl, kWave - 1);
  }
  const double loc = use_p ? lp : lw;
  const double t = u24(philox_at(seed, static_cast<uint32_t>(n), static_cast<uint32_t>(r)).y) * W;
  // this lane's sub-chunks from running weight run0: the first whose running
  // weight exceeds t (first_over), or the last with positive weight
  auto search = [&](double run0, bool first_over, int& found, double& fb) {
    double run = run0;
#pragma unroll
    for (int k = 0; k < kPickCache; ++k) {
      const int s = s0 + k;
      const double ws = use_p ? cp_[k] : cw_[k];
      if (s < s1) {
        if (first_over ? (found < 0 && run + ws > t) : ws > 0.0) {
          found = s;
          fb = run;
        }
        run += ws;
      }
    }
    for (int s = s0 + kPickCache; s < s1; ++s) {
      const double ws = subp[2 * s + (use_p ? 1 : 0)];
      if (first_over ? (found < 0 && run + ws > t) : ws > 0.0) {
        found = s;
        fb = run;
      }
      run += ws;
    }
  };
  int sub = -1;
  double base = 0.0;
  const uint64_t over = __ballot(incl > t);
  if (over) {
    const int L = __ffsll(static_cast<long long>(over)) - 1;
    int found = -1;
    double fb = 0.0;
    if (lane == L) {
      search(incl - loc, true, found, fb);
      if (found < 0) search(incl - loc, false, found, fb);  // rounding inside the lane
    }
    sub = bcast_i32(found, L);
    base = bcast_f64(fb, L);
  }
  if (sub < 0) {  // rounding: the last sub-chunk with positive weight
    int last = -1;
    double lb = 0.0;
    search(incl - loc, false, last, lb);
    const int lmax = wave_max_i32(last);
    if (lmax >= 0) {
      const uint64_t who = __ballot(last == lmax);
      const int L = __ffsll(static_cast<long long>(who)) - 1;
      sub = lmax;
      base = bcast_f64(lb, L);
    } else {
      sub = 0;
      base = 0.0;
    }
  }
  // the sub-chunk: lane = 8-value group
  const int g = sub * kSubG + lane;
  const bool in = g < groups_of(a.V);
  const bool dense_res = kDense && !use_p;
  double w8[8];
  {
    float l[8], d[8];
    if (in) {
      load8(row_ptr(a.tgt, a.dtype, rec.trow, a.tgt_ld), a.dtype, g, a.V, l);
      if (dense_res) load8(row_ptr(a.draft, a.ddtype, rec.drow, a.draft_ld), a.ddtype, g, a.V, d);
    }
    const float cut = rec.cut;
    const double invT = rec.invT, kept = rec.kept, dlse = rec.dlse;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      double w = 0.0;
      if (in && g * 8 + q < a.V) {
        w = p_of(l[q], cut, invT, kept);
        if (dense_res) {
          const double t2 = w - exp(static_cast<double>(d[q]) * invT - dlse);
          w = t2 > 0.0 ? t2 : 0.0;
        }
      }
      w8[q] = w;
    }
  }
  if (!kDense && !use_p) {
    const int nc = rec.ncorr;
    for (int t2 = 0; t2 < nc; ++t2) {
      const int v = bcast_i32(ctok, t2);
      const double wv = bcast_f64(cwt, t2);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (v == g * 8 + q) w8[q] = wv;
    }
  }
  double lsum = 0.0;
#pragma unroll
  for (int q = 0; q < 8; ++q) lsum += w8[q];
  const double inc2 = wave_incl_scan_f64(lsum);
  const uint64_t hit = __ballot(in && base + inc2 > t);
  int lastpos = -1;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (w8[q] > 0.0) lastpos = g * 8 + q;
  int tok;
  if (hit) {
    const int L = __ffsll(static_cast<long long>(hit)) - 1;
    int pick = -1;
    double acc = base + inc2 - lsum;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      acc += w8[q];
      if (acc > t && pick < 0 && w8[q] > 0.0) pick = g * 8 + q;
    }
    if (pick < 0) pick = lastpos;
    tok = bcast_i32(pick, L);
    if (tok < 0) tok = wave_max_i32(lastpos);
  } else {  // rounding: the last positive weight of the sub-chunk
    tok = wave_max_i32(lastpos);
  }
  if (tok < 0) tok = sub * kSubG * 8;
  if (lane == 0) {
    a.token[r] = tok;
    a.is_bonus[r] = bonus;
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
  a.rec = reinterpret_cast<DrawRec*>(static_cast<char*>(ws) + l.rec);
  a.sub = reinterpret_cast<double*>(static_cast<char*>(ws) + l.sub);
  a.NSUB = sub_chunks(V);
  a.S = res_chunks(V);
  return a;
}

// sums grid, then the pick; dynamic LDS holds the mixture's branch tables
template <bool kDense, bool kAccept>
static int32_t launch_draw(const SampleArgs& a, hipStream_t s) {
  const size_t dyn = kDense ? 0 : sizeof(int) * 2 * static_cast<size_t>(a.K) * a.b;
  hipLaunchKernelGGL((k_draw_sums<kDense, kAccept>), dim3(a.R * a.S), dim3(kSumNT), dyn, s, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  hipLaunchKernelGGL(k_pick<kDense>, dim3(a.R), dim3(kWave), 0, s, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
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
  return q_mode == SV_Q_DENSE ? launch_draw<true, false>(a, s) : launch_draw<false, false>(a, s);
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
  return q_mode == SV_Q_DENSE ? launch_draw<true, true>(a, s) : launch_draw<false, true>(a, s);
}
