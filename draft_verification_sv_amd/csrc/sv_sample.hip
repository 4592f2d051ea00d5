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

#include <mutex>

#include "sv_device.hpp"
#include "sv_draw.hpp"
#include "sv_host.hpp"

namespace sv {

// target probability of a token with logit l: [l >= cut] exp(l / T - kept_lse), T > 0
// (tab: the exponential's table, exp_table_init)
__device__ __forceinline__ double p_of(float l, float cut, double invT, double kept, const double* tab) {
  return l >= cut ? exp_tab(static_cast<double>(l) * invT - kept, tab) : 0.0;
}

// One element's raw bits (bf16: the 16-bit pattern; fp32: the word), converted
// later by raw_f32, so that a load inside a branch needs no wait there.
template <int DT>
__device__ __forceinline__ uint32_t raw1(const char* rowp, int idx) {
  if constexpr (DT == SV_BF16) return reinterpret_cast<const uint16_t*>(rowp)[idx];
  else return reinterpret_cast<const uint32_t*>(rowp)[idx];
}
template <int DT>
__device__ __forceinline__ float raw_f32(uint32_t w) {
  return __uint_as_float(DT == SV_BF16 ? w << 16 : w);
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
__device__ __forceinline__ int accept_wave(const SampleArgs& a, int r, int pb, int Lr, int tb, const double* qx,
                                           const double* tab) {
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
        p = p_of(l, a.row_cut[trow], invT, a.row_kept[trow], tab);
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
          q = exp_tab(static_cast<double>(d) * invT - a.dlse[pos], tab);
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
  __shared__ double etab[kExpTab];
  exp_table_init(etab);
  __syncthreads();
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
  const int n = accept_wave(a, r, pb, Lr, tb, qx, etab);
  if (threadIdx.x == 0) a.n_acc[r] = n;
}

// ------------------------------------------------------------------ the draw
// What the chunk blocks of one request share (built by wave 0).
struct DrawCtx {
  int mode, n, bonus, token, ncorr;
  float cut;
  double invT, kept, dlse, invTb;
  int64_t trow, drow;
  int ctok[64];
  double cq[64];  // greedy-branch residual: q at ctok
  double cw[64];  // soft branches: lse_z - log w_z per branch z
};

struct TailShared {
  // A. draft tokens and mixing logits
  int x[64];
  float mix[64];
  // B. statistics of the candidate rows tb + i (i <= L_r); the mixture's
  // q(z | y) and f_z (the first position where branch z leaves the draft)
  float rc[65];
  double rk[65];
  int ra[65];
  double pi[64];
  int f[64];
  // standalone draw: branch tokens and posterior weights at the slot
  int tv[64];
  double tw[64];
  double mrow[65];  // soft tail: maximum of each position's log posterior
  double etab[kExpTab];  // the exponential's table
  DrawCtx c;
};

// D's per-wave lists of values at or above the cut: the kLists sub-chunks of
// a pass are packed one after another into one list (then one dummy slot per
// lane), so that exp runs over the pass's kept values with no idle slots.  The
// lists share the dynamic LDS with the mixture's branch tables, which are dead
// by then.  Dense proposals keep one sub-chunk per pass (two lists of it, p
// and q): 18 KiB of lists, so that six blocks fit on a compute unit and the
// grid of 32 requests at V = 151936 (1216 blocks) is resident at once; two sub-chunks per pass
// took 34 KiB, four blocks per compute unit and a second round of blocks.
template <bool kDense>
struct DLists {
  static constexpr int kLists = (kDense ? 1 : 4) < kSubPerWave ? (kDense ? 1 : 4) : kSubPerWave;  // sub-chunks per pass
  static constexpr int kCap = kLists * kSubG * 8;                        // values of a pass
  static constexpr int kPerWave = (kCap + kWave) * (kDense ? 2 : 1);     // floats
  static constexpr size_t kBytes = sizeof(float) * kPerWave * (kSumNT / kWave);
};

// Mixture residual at the draw slot (wave 0): lane z < K holds branch z (whether
// it is consistent with the accepted prefix, its token v and its posterior
// weight w).  q(v) is the summed weight of the branches with token v; the draw
// weight at v is max(0, p(v) - q(v)), formed by the kernels that read v's
// logit with the rest of its sub-chunk; every other token keeps p.  The
// distinct tokens and their q go to c.ctok, c.cq in lane order.
__device__ __forceinline__ void build_corrections(DrawCtx& c, int K, bool act, int v, double w) {
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
    c.ctok[idx] = v;
    c.cq[idx] = q;
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
    d.invTb = c.invTb;
  }
  if (lane < c.ncorr) {
    d.ctok[lane] = c.ctok[lane];
    d.cw[lane] = c.cw[lane];
    d.cq[lane] = c.cq[lane];
  }
}

// A(i) = sum_z pi_z [f_z >= i] and A(i + 1), lane i (pi, f in LDS, K <= 64).
__device__ __forceinline__ void posterior_mass(const TailShared& sh, int K, int i, double& Ai, double& Ai1) {
  Ai = 0.0;
  Ai1 = 0.0;
#pragma unroll 8
  for (int z = 0; z < K; ++z) {
    const double pz = sh.pi[z];
    const int fz = sh.f[z];
    Ai += fz >= i ? pz : 0.0;
    Ai1 += fz > i ? pz : 0.0;
  }
}

// Value e (0..7) of the 8-value group that lane src of the wave loaded as raw
// words (w0, w1 as raw8 loads them); every lane of the wave calls it.
template <int DT>
__device__ __forceinline__ float value_from_lane(const uint4& w0, const uint4& w1, int src, int e) {
  const uint32_t a0 = __shfl(w0.x, src), a1 = __shfl(w0.y, src), a2 = __shfl(w0.z, src), a3 = __shfl(w0.w, src);
  if constexpr (DT == SV_BF16) {
    const int wi = e >> 1;
    const uint32_t w = wi == 0 ? a0 : wi == 1 ? a1 : wi == 2 ? a2 : a3;
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    const uint32_t b0 = __shfl(w1.x, src), b1 = __shfl(w1.y, src), b2 = __shfl(w1.z, src), b3 = __shfl(w1.w, src);
    const int wi = e & 3;
    const uint32_t lo = wi == 0 ? a0 : wi == 1 ? a1 : wi == 2 ? a2 : a3;
    const uint32_t hi = wi == 0 ? b0 : wi == 1 ? b1 : wi == 2 ? b2 : b3;
    return __uint_as_float(e < 4 ? lo : hi);
  }
}

// D. Sums of p and of the draw weight over the sub-chunks of chunk ch of the
// drawn row; wave wv takes sub-chunks ch*16 + k*4 + wv, k < 4, one 8-value
// group per lane, all loaded before any arithmetic.  Only values at or above
// the top-p cut carry weight: kLists sub-chunks at a time, each sub-chunk's
// such values are packed densely into a list (positions from a wave scan of the
// per-lane counts; the other values go to the lane's dummy slot, so no store
// branches), then exp runs over the lists, interleaved.
template <int DT, int DDT, bool kDense>
__device__ __forceinline__ void sub_sums(const SampleArgs& a, const DrawCtx& c, int r, int ch, float* lists,
                                         const double* tab) {
  using DL = DLists<kDense>;
  constexpr int kL = DL::kLists, kLen = kSubG * 8;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int V = a.V, NG = groups_of(V);
  const bool dense_res = kDense && c.mode == kDrawResidual;
  const bool mix_res = !kDense && c.mode == kDrawResidual;
  const float cut = c.cut;
  const double invT = c.invT, kept = c.kept, dlse = c.dlse;
  const char* trowp = row_ptr(a.tgt, DT, c.trow, a.tgt_ld);
  const char* drowp = kDense ? row_ptr(a.draft, DDT, c.drow, a.draft_ld) : nullptr;
  float* st = lists + wv * DL::kPerWave;  // the pass's kept target values, then lane dummies
  float* sd = st + DL::kCap + kWave;      // dense: the matching draft values
  const int sub0 = ch * kChunkSubs + wv;
  uint4 t0[kSubPerWave], t1[kSubPerWave], d0[kSubPerWave], d1[kSubPerWave];
#pragma unroll
  for (int k = 0; k < kSubPerWave; ++k) {
    const int g = min((sub0 + k * (kSumNT / kWave)) * kSubG + lane, NG - 1);
    raw8<DT>(trowp, g, V, t0[k], t1[k]);
    if (dense_res) raw8<DDT>(drowp, g, V, d0[k], d1[k]);
  }
  // corrections of the mixture residual: lane t < ncorr holds branch token t
  const int ctok = mix_res && lane < c.ncorr ? c.ctok[lane] : -1;
  const double cq = mix_res && lane < c.ncorr ? c.cq[lane] : 0.0;
  // one sub-chunk (the k-th of the wave)'s two sums, the branch-token
  // corrections added, by lane 0
  auto publish = [&](int sub, int k, double sp, double sw) {
    const double tp = wave_sum_f64(sp);
    double tw = dense_res ? wave_sum_f64(sw) : tp;
    if (mix_res) {  // branch tokens in this sub-chunk: weight max(0, p - q) instead of p
      const int v0 = sub * kLen;
      const bool here = ctok >= v0 && ctok < v0 + kLen && ctok < V;
      if (__ballot(here)) {  // p at the token, from the lane that loaded its group
        const int o = here ? ctok - v0 : 0;
        const double p = p_of(value_from_lane<DT>(t0[k], t1[k], o >> 3, o & 7), cut, invT, kept, tab);
        const double d = p - cq;
        tw += wave_sum_f64(here ? (d > 0.0 ? d : 0.0) - p : 0.0);
      }
    }
    if (lane == 0) {
      double* pp = a.sub + (static_cast<size_t>(r) * a.NSUB + sub) * 2;
      pp[0] = tw;
      pp[1] = tp;
    }
  };
  if (cut == -INFINITY) {  // no cut: every value weighs; sums straight from the registers
#pragma unroll
    for (int k = 0; k < kSubPerWave; ++k) {
      const int sub = sub0 + k * (kSumNT / kWave);
      if (sub >= a.NSUB) break;  // wave-uniform
      const int g = sub * kSubG + lane;
      const int valid = g < NG ? min(V - g * 8, 8) : 0;
      float l[8], d[8];
      unpack8<DT>(t0[k], t1[k], l);
      if (dense_res) unpack8<DDT>(d0[k], d1[k], d);
      double sp = 0.0, sw = 0.0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool keep = q < valid && l[q] >= cut;  // NaN and values past the row weigh 0
        const double p = exp_tab(keep ? static_cast<double>(l[q]) * invT - kept : -INFINITY, tab);
        sp += p;
        if (dense_res) {
          const double t = p - exp_tab(keep ? static_cast<double>(d[q]) * invT - dlse : -INFINITY, tab);
          sw += t > 0.0 ? t : 0.0;
        }
      }
      publish(sub, k, sp, sw);
    }
    return;
  }
#pragma unroll
  for (int k0 = 0; k0 < kSubPerWave; k0 += kL) {
    if (sub0 + k0 * (kSumNT / kWave) >= a.NSUB) break;  // wave-uniform
    // pack: segment j holds sub-chunk k0 + j's kept values, in vocabulary order
    int seg[kL + 1];
    seg[0] = 0;
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      const int k = k0 + j;
      const int g = (sub0 + k * (kSumNT / kWave)) * kSubG + lane;
      const int valid = g < NG ? min(V - g * 8, 8) : 0;
      float l[8], d[8];
      unpack8<DT>(t0[k], t1[k], l);
      if (dense_res) unpack8<DDT>(d0[k], d1[k], d);
      if (valid < 8)  // the row's last group, or past its end: those values are dropped
#pragma unroll
        for (int q = 0; q < 8; ++q) l[q] = q < valid ? l[q] : -INFINITY;
      int cnt = 0;  // -inf fails the test unless the cut is -inf (then it weighs 0)
#pragma unroll
      for (int q = 0; q < 8; ++q) cnt += l[q] >= cut ? 1 : 0;
      const int inc = wave_incl_scan_i32(cnt);
      int o = seg[j] + inc - cnt;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool keep = l[q] >= cut;
        const int at = keep ? o : DL::kCap + lane;
        st[at] = l[q];
        if (dense_res) sd[at] = d[q];
        o += keep ? 1 : 0;
      }
      seg[j + 1] = seg[j] + bcast_i32(inc, kWave - 1);
    }
    __syncwarp();
    double sp[kL], sw[kL];
#pragma unroll
    for (int j = 0; j < kL; ++j) sp[j] = sw[j] = 0.0;
    for (int e = lane; e < seg[kL]; e += kWave) {
      const double p = exp_tab(static_cast<double>(st[e]) * invT - kept, tab);
      double t = 0.0;
      if (dense_res) {
        t = p - exp_tab(static_cast<double>(sd[e]) * invT - dlse, tab);
        t = t > 0.0 ? t : 0.0;
      }
#pragma unroll
      for (int j = 0; j < kL; ++j) {  // the segment holding e
        const bool here = e >= seg[j] && e < seg[j + 1];
        sp[j] += here ? p : 0.0;
        if (dense_res) sw[j] += here ? t : 0.0;
      }
    }
    __syncwarp();  // the list is rewritten by the next pass
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      const int sub = sub0 + (k0 + j) * (kSumNT / kWave);
      if (sub >= a.NSUB) break;  // wave-uniform
      publish(sub, k0 + j, sp[j], sw[j]);
    }
  }
}

// The fused tail (kAccept: posterior, acceptance and the draw's sums) or the
// standalone draw's sums (n from n_acc_in, posterior weights from post_w).
// DT / DDT: target / dense-draft logit types.
template <int DT, int DDT, bool kDense, bool kAccept>
__global__ __launch_bounds__(kSumNT) void k_draw_sums(SampleArgs a) {
  __shared__ TailShared sh;
  // dynamic LDS: the mixture's branch tokens [K][b] through phase C, then D's lists
  extern __shared__ __align__(16) int dyn[];
  int* g = dyn;
  const int r = blockIdx.x / a.S, ch = blockIdx.x % a.S;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const bool report = ch == 0;
  const int K = kDense ? 0 : a.K, b = a.b, V = a.V;
  DrawCtx& c = sh.c;

  // A. the request header (uniform: scalar loads) and the draft tokens, mixing
  // logits and branch tokens (one per thread, clamped in-bounds), all issued
  // before any is used; the offsets are checked after the barrier.  Also the
  // statistics of target row i = thread (i <= b, clamped) and the logit at
  // its draft token, and for a dense draft its row's lse, argmax and logit at
  // the token, from the rows launch's slot records: they need no offset, so
  // no load waits for another.
  const int pb = a.pos_off[r], pe = a.pos_off[r + 1], tb = a.tgt_off[r], te = a.tgt_off[r + 1];
  const float T = a.T[r];
  const int nin = kAccept ? 0 : a.n_acc_in[r];
  int x0 = 0;
  float m0 = 0.0f;
  uint64_t k0[kMixParts];  // the parts of branch (z, i) = thread t: the argmax is the largest key
#pragma unroll
  for (int q = 0; q < kMixParts; ++q) k0[q] = 0;
  const uint64_t* kr = a.bkey + static_cast<size_t>(r) * K * b * kMixParts;
  float s_cut = 0.0f, s_lx = 0.0f, s_dx = 0.0f;
  double s_kept = 0.0, s_dl = 0.0;
  int s_arg = 0, s_da = 0;
  uint64_t seed = 0;
  if (kAccept) {
    x0 = a.x[static_cast<size_t>(r) * b + min(tid, b - 1)];
    if (!kDense) {
      m0 = a.mix[static_cast<size_t>(r) * K + min(tid, K - 1)];
#pragma unroll
      for (int q = 0; q < kMixParts; ++q) k0[q] = kr[static_cast<size_t>(min(tid, K * b - 1)) * kMixParts + q];
    } else {
      const SlotRec& dr = a.dslot[static_cast<size_t>(r) * (b + 1) + min(tid, b - 1)];
      s_dl = dr.kept;
      s_da = dr.argmax;
      s_dx = dr.lx;
    }
    const SlotRec& sr = a.slot[static_cast<size_t>(r) * (b + 1) + min(tid, b)];
    s_cut = sr.cut;
    s_kept = sr.kept;
    s_arg = sr.argmax;
    s_lx = sr.lx;
    seed = *a.seed;
  }
  asm volatile("" ::: "memory");  // the compiler keeps every load above ahead of what follows
  exp_table_init(sh.etab);
  auto merged = [&](const uint64_t* ks) -> int {
    uint64_t m = 0;
#pragma unroll
    for (int q = 0; q < kMixParts; ++q) m = ks[q] > m ? ks[q] : m;
    return static_cast<int>(argmax_token(m));
  };
  if (tid < kWave) sh.f[tid] = 0x7FFFFFFF;
  if (kAccept) {
    if (tid < b) sh.x[tid] = x0;
    if (!kDense) {
      if (tid < K) sh.mix[tid] = m0;
      if (tid < K * b) g[tid] = merged(k0);
      for (int k = tid + kSumNT; k < K * b; k += kSumNT) {  // K * b > kSumNT only
        uint64_t ks[kMixParts];
#pragma unroll
        for (int q = 0; q < kMixParts; ++q) ks[q] = kr[static_cast<size_t>(k) * kMixParts + q];
        g[k] = merged(ks);
      }
    }
  }
  __syncthreads();
  const int Lr = pe - pb;
  if (!(Lr >= 0 && Lr <= b && te - tb == Lr + 1)) {
    if (report && tid == 0) {
      raise_status(a.status, SV_ST_BAD_OFFSETS);
      if (kAccept) a.n_acc[r] = 0;
      a.rec[r].mode = kDrawNone;
    }
    return;
  }
  const bool greedy = T == 0.0f;
  const double invT = 1.0 / static_cast<double>(T);

  if (kAccept) {
    // B. everything from phase A's loads (the slot records); mixture: f_z by
    // LDS atomicMin.  Thread i (< L_r) keeps p(x_i), the dense q(x_i) and u_i
    // in registers for phase C; wave 1 forms q(z | y).
    const int xl = x0;  // thread i < L_r loaded x_i itself
    const bool xok = xl >= 0 && xl < V;
    const float rc0 = s_cut, lxv = s_lx;
    const double rk0 = s_kept, dl0 = s_dl;
    const int ra0 = s_arg, da0 = s_da;
    const int KL = K * Lr, Lq = Lr > 0 ? Lr : 1;
    if (!kDense) {  // clamped in-bounds also when K * L_r = 0
      const int k = min(tid, KL > 0 ? KL - 1 : 0);
      const int gz = k / Lq, gi = k - gz * Lq;
      if (tid < KL && g[gz * b + gi] != sh.x[gi]) atomicMin(&sh.f[gz], gi);
    }
    if (!kDense && report)  // the merged branch argmax, i < L_r
      for (int k = tid; k < K * b; k += kSumNT)
        if (k % b < Lr) a.branch_out[static_cast<size_t>(r) * K * b + k] = g[k];
    if (tid <= Lr) {
      sh.rc[tid] = rc0;
      sh.rk[tid] = rk0;
      sh.ra[tid] = ra0;
    }
    if (!kDense) {
      for (int k = tid + kSumNT; k < KL; k += kSumNT) {  // K * L_r > kSumNT only
        const int z = k / Lr, i = k - z * Lr;
        if (g[z * b + i] != sh.x[i]) atomicMin(&sh.f[z], i);
      }
      if (wv == 1) {  // q(z | y) = softmax of the mixing logits
        const bool act = lane < K;
        const float ml = act ? sh.mix[lane] : -INFINITY;
        const float mmax = wave_max_f32(ml);
        const double e = act ? exp(static_cast<double>(ml) - static_cast<double>(mmax)) : 0.0;
        sh.pi[lane] = e / wave_sum_f64(e);
      }
    }
    // lane i < L_r of wave 0: p(x_i), the dense q(x_i), u_i (word 0)
    const bool pos = tid < Lr;
    double p = 0.0, qd = 0.0, u = 0.0;
    if (tid < kWave) {
      u = u24(philox_at(seed, static_cast<uint32_t>(lane), static_cast<uint32_t>(r)).x);
      if (pos && xok) {
        p = greedy ? (xl == ra0 ? 1.0 : 0.0) : p_of(lxv, rc0, invT, rk0, sh.etab);
        if (kDense)
          qd = greedy ? (xl == da0 ? 1.0 : 0.0) : exp_tab(static_cast<double>(s_dx) * invT - dl0, sh.etab);
      }
      if (report && pos && !xok) raise_status(a.status, SV_ST_BAD_TOKEN);
    }
    __syncthreads();

    // C. acceptance and the draw context (wave 0); posterior outputs (wave 1 of
    // the reporting block)
    if (tid < kWave) {
      double q = qd, A = 0.0;  // lane i: q(x_i | x_<i), A(i)
      if (!kDense) {
        // w_z^(i) = pi_z [f_z >= i] / A(i), q(x_i | x_<i) = A(i + 1) / A(i)
        double Ai1;
        posterior_mass(sh, K, lane, A, Ai1);
        q = pos && xok && A > 0.0 ? Ai1 / A : 0.0;
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
      const double dln = kDense ? bcast_f64(dl0, n < Lr ? n : 0) : 0.0;  // lane n loaded slot n's lse
      if (lane == 0) {
        c.n = n;
        c.bonus = n == Lr ? 1 : 0;
        c.mode = greedy ? kDrawGreedy : (n == Lr ? kDrawP : kDrawResidual);
        c.token = sh.ra[n];
        c.cut = sh.rc[n];
        c.kept = sh.rk[n];
        c.invT = invT;
        c.dlse = kDense && n < Lr ? dln : 0.0;
        c.trow = tb + n;
        c.drow = static_cast<int64_t>(r) * b + n;
        c.ncorr = 0;
        c.invTb = 0.0;
      }
      __syncwarp();
      if (!kDense && !greedy && n < Lr) {
        const double An = bcast_f64(A, n);
        const int f = lane < K ? min(sh.f[lane], Lr) : -1;
        const bool act = lane < K && f >= n;
        build_corrections(c, K, act, act ? g[lane * b + n] : -1, act ? sh.pi[lane] / An : 0.0);
      }
      __syncwarp();
      if (report) write_record(a, r, c);
    } else if (!kDense && report && wv == 1) {
      // post_w[i][z] and q_at_draft[i], lane i < L_r
      double Ai, Ai1;
      posterior_mass(sh, K, lane, Ai, Ai1);
      if (lane < Lr) {
        a.q_at_draft[static_cast<size_t>(r) * b + lane] = Ai > 0.0 ? Ai1 / Ai : 0.0;
        if (!(Ai > 0.0)) raise_status(a.status, SV_ST_EMPTY_POSTERIOR);
        double* pw = a.post_w + (static_cast<size_t>(r) * b + lane) * K;
        for (int z = 0; z < K; ++z) pw[z] = Ai > 0.0 && min(sh.f[z], Lr) >= lane ? sh.pi[z] / Ai : 0.0;
      }
    }
  } else {
    // standalone draw: n given; branch tokens and posterior weights at slot n given
    int n = nin;
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
      c.invTb = 0.0;
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
        build_corrections(c, K, in && w > 0.0 && v >= 0 && v < V, v, w);
      }
      __syncwarp();
      if (report) write_record(a, r, c);
    }
  }
  __syncthreads();  // also ends every use of the branch tables, which D's lists overwrite
  if (c.mode == kDrawGreedy) return;  // the draw is the argmax (taken by the pick kernel)
  sub_sums<DT, DDT, kDense>(a, c, r, ch, reinterpret_cast<float*>(dyn), sh.etab);
}

// ------------------------------------------------------------------ soft branches
// Branch z's distribution at position i is softmax(c_{z,i} / T_b) ("Pith review
// of DBLAST", "What carries the argument": q_dep = sum_z q(z|y) prod_i
// q_i(x_i | y, z)).  By Bayes' rule on the mixture the category posterior
// before position i is proportional to q(z|y) prod_{j<i} q_j(x_j | z), carried
// in logs and normalised per position; q(x_i | x_<i) = sum_z w_z q_i(x_i | z).
// A rejection at j draws from norm(max(0, p_j - sum_z w_z q_j(. | z))), which
// reads the K branch rows of slot j next to the target row.  A request with
// T_b = 0 keeps point-mass branches at each row's argmax (the greedy residual).

// p and the soft-residual weight of the 8 values of group g of the drawn row:
// max(0, p(v) - sum_z exp(c_z(v) / T_b - off_z)), off_z = lse_z - log w_z
// (+inf where w_z = 0); the branch sum is formed only where p(v) > 0.  Branch
// z's row is crow0 + z * cstride bytes.
template <int DT>
__device__ __forceinline__ void soft_group(const SampleArgs& a, const char* trowp, const char* crow0, size_t cstride,
                                           const double* off, int g, float cut, double invT, double kept,
                                           double invTb, const double* tab, double p8[8], double w8[8]) {
  constexpr int kB = 8;  // branch rows whose 16-byte words are in flight together
  const int V = a.V, NG = groups_of(V), K = a.K;
  const int gc = min(g, NG - 1);
  uint4 t0, t1, c0[kB], c1[kB];
  raw8<DT>(trowp, gc, V, t0, t1);
#pragma unroll
  for (int j = 0; j < kB; ++j) raw8<DT>(crow0 + cstride * min(j, K - 1), gc, V, c0[j], c1[j]);
  asm volatile("" ::: "memory");  // every load above is issued before any is used
  float l[8];
  decode8<DT>(t0, t1, g, V, g < NG, l);
  double q8[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    p8[q] = l[q] > -INFINITY ? p_of(l[q], cut, invT, kept, tab) : 0.0;
    q8[q] = 0.0;
  }
  for (int z0 = 0; z0 < K; z0 += kB) {
    if (z0 > 0) {  // K > 8 only
#pragma unroll
      for (int j = 0; j < kB; ++j) raw8<DT>(crow0 + cstride * min(z0 + j, K - 1), gc, V, c0[j], c1[j]);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const double o = off[min(z0 + j, K - 1)];
      if (z0 + j < K && o < INFINITY) {
        float cv[8];
        unpack8<DT>(c0[j], c1[j], cv);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (p8[q] > 0.0) q8[q] += exp_tab(static_cast<double>(cv[q]) * invTb - o, tab);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const double t = p8[q] - q8[q];
    w8[q] = t > 0.0 ? t : 0.0;
  }
}

// D (soft residual): sums of p and of the draw weight over sub-chunk `sub`
// (one group per lane) by one wave.
template <int DT>
__device__ __forceinline__ void sub_sum_soft(const SampleArgs& a, const DrawCtx& c, int r, int sub, const double* tab) {
  const int lane = threadIdx.x & (kWave - 1);
  const char* trowp = row_ptr(a.tgt, DT, c.trow, a.tgt_ld);
  const char* crow0 = row_ptr(a.comp, DT, c.drow, a.comp_ld);
  const size_t cstride = static_cast<size_t>(a.b) * static_cast<size_t>(a.comp_ld) * (DT == SV_BF16 ? 2 : 4);
  double p8[8], w8[8];
  soft_group<DT>(a, trowp, crow0, cstride, c.cw, sub * kSubG + lane, c.cut, c.invT, c.kept, c.invTb, tab, p8, w8);
  double sp = 0.0, sw = 0.0;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    sp += p8[q];
    sw += w8[q];
  }
  const double tp = wave_sum_f64(sp), tw = wave_sum_f64(sw);
  if (lane == 0) {
    double* pp = a.sub + (static_cast<size_t>(r) * a.NSUB + sub) * 2;
    pp[0] = tw;
    pp[1] = tp;
  }
}

// D (soft residual, bf16 rows, K <= kSoftB): the same sums over the values of
// the nucleus only.  The wave stores its 64 target words and the K branch
// words of the sub-chunk in LDS and packs the positions at or above the cut
// into a list (wave scan of per-lane counts), so that the K exponentials per
// value run over kept values with no idle lanes (about a fifth of a sub-chunk
// at top-p 0.95).  Per value the terms are formed exactly as in soft_group
// (branches in ascending order), so the pick kernel re-forms the same weights.
constexpr int kSoftB = 8;  // branch rows per pass of soft_group; the list path takes K <= kSoftB
struct SoftLists {
  static constexpr size_t kPerWave = static_cast<size_t>(kSoftB + 1) * kWave * 16 + kSubG * 8 * sizeof(uint16_t);
  static constexpr size_t kBytes = kPerWave * (kSumNT / kWave);
};

// Calls f(i, p, w) for every value i of sub-chunk `sub` at or above the cut,
// by one wave (lane-strided over the packed list); `lds` is the wave's
// SoftLists::kPerWave bytes.
template <typename F>
__device__ __forceinline__ void soft_nucleus(const SampleArgs& a, const char* trowp, const char* crow0,
                                             size_t cstride, const double* off, int sub, float cut, double invT,
                                             double kept, double invTb, const double* tab, char* lds, F&& f) {
  const int lane = threadIdx.x & (kWave - 1);
  u32x4_t* words = reinterpret_cast<u32x4_t*>(lds);  // [1 + kSoftB][kWave], target first
  uint16_t* pos = reinterpret_cast<uint16_t*>(words + (kSoftB + 1) * kWave);
  const uint16_t* vals = reinterpret_cast<const uint16_t*>(words);  // value i of row j at j * 512 + i
  const int V = a.V, NG = groups_of(V), K = a.K;
  const int g = sub * kSubG + lane, gc = min(g, NG - 1);
  // 16-byte words as native vectors (kept in registers), all loads issued before any is used
  const u32x4_t tword = *reinterpret_cast<const u32x4_t*>(trowp + static_cast<size_t>(gc) * 16);
  u32x4_t cw[kSoftB];
#pragma unroll
  for (int j = 0; j < kSoftB; ++j)
    cw[j] = *reinterpret_cast<const u32x4_t*>(crow0 + cstride * min(j, K - 1) + static_cast<size_t>(gc) * 16);
  asm volatile("" ::: "memory");
  words[lane] = tword;
#pragma unroll
  for (int j = 0; j < kSoftB; ++j) words[(1 + j) * kWave + lane] = cw[j];  // rows past K repeat row K - 1, unread
  const uint4 t0 = {tword.x, tword.y, tword.z, tword.w};
  float l[8];
  decode8<SV_BF16>(t0, t0, g, V, g < NG, l);  // values past the row read -inf
  int cnt = 0;  // p > 0 only at or above the cut; -inf and NaN weigh 0
#pragma unroll
  for (int q = 0; q < 8; ++q) cnt += l[q] >= cut && l[q] > -INFINITY ? 1 : 0;
  const int inc = wave_incl_scan_i32(cnt);
  const int n = bcast_i32(inc, kWave - 1);
  int o = inc - cnt;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    if (l[q] >= cut && l[q] > -INFINITY) pos[o++] = static_cast<uint16_t>(lane * 8 + q);
  __syncwarp();
  for (int e = lane; e < n; e += kWave) {
    const int i = pos[e];
    const double p = exp_tab(static_cast<double>(__uint_as_float(static_cast<uint32_t>(vals[i]) << 16)) * invT - kept, tab);
    double qv = 0.0;
#pragma unroll
    for (int j = 0; j < kSoftB; ++j) {
      const double oz = off[min(j, K - 1)];
      if (j < K && oz < INFINITY)
        qv += exp_tab(static_cast<double>(__uint_as_float(static_cast<uint32_t>(vals[(1 + j) * kSubG * 8 + i]) << 16)) *
                          invTb - oz,
                      tab);
    }
    const double t = p - qv;
    f(i, p, t > 0.0 ? t : 0.0);
  }
  __syncwarp();  // the wave's list and words may be rewritten by its next sub-chunk
}

__device__ __forceinline__ void sub_sum_soft_lists(const SampleArgs& a, const DrawCtx& c, int r, int sub,
                                                   const double* tab, char* lds) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const size_t cstride = static_cast<size_t>(a.b) * static_cast<size_t>(a.comp_ld) * 2;
  double sp = 0.0, sw = 0.0;
  soft_nucleus(a, row_ptr(a.tgt, SV_BF16, c.trow, a.tgt_ld), row_ptr(a.comp, SV_BF16, c.drow, a.comp_ld), cstride,
               c.cw, sub, c.cut, c.invT, c.kept, c.invTb, tab, lds + wv * SoftLists::kPerWave,
               [&](int, double p, double w) {
                 sp += p;
                 sw += w;
               });
  const double tp = wave_sum_f64(sp), tw = wave_sum_f64(sw);
  if (lane == 0) {
    double* pp = a.sub + (static_cast<size_t>(r) * a.NSUB + sub) * 2;
    pp[0] = tw;
    pp[1] = tp;
  }
}

// Dynamic LDS of the soft tail: branch argmax [K][b] (int), log q_i(x_i | z)
// [K][b], the branch rows' lse [K][b] and the unnormalised log posterior
// [b + 1][K] (double); D's lists reuse it.
constexpr long long kSoftMaxKb = 2048;  // K * b bound of the soft tail (its tables stay below 60 KB)

__host__ __device__ inline size_t soft_tables_bytes(int K, int b) {
  const size_t kb = static_cast<size_t>(K) * b;
  return sizeof(int) * ((kb + 1) & ~static_cast<size_t>(1)) + 2 * sizeof(double) * kb +
         sizeof(double) * static_cast<size_t>(b + 1) * K;
}

// Blocks per request of the soft tail: kSoftSubs sub-chunks per wave, so that
// a soft chunk is one chunk of the greedy tail (a p or greedy-branch draw in
// soft mode then sums that chunk).
constexpr int kSoftSubs = 2;
constexpr int kSoftChunk = (kSumNT / kWave) * kSoftSubs;  // sub-chunks of a soft chunk
static_assert(kSoftChunk == kChunkSubs, "a soft chunk is one greedy chunk");
__host__ __device__ inline int soft_chunks(int V) { return (sub_chunks(V) + kSoftChunk - 1) / kSoftChunk; }

// The fused tail with soft branches, first launch (one block per request): A
// and B load the header, the draft tokens, the mixing logits, the branch
// argmax and lse of the rows launch and every branch's logit at the draft
// tokens; C1 forms the posterior's exponentials, one (position, branch) per
// thread; C (wave 0) runs the acceptance tests and writes the draw record.
// The sums over the drawn row (k_soft_body) read only that record: with K
// branch rows per value they are long enough that recomputing A-C in each of
// their blocks, as the greedy tail does, would hold every block up before its
// first load.
template <int DT>
__global__ __launch_bounds__(kSumNT) void k_soft_head(SampleArgs a) {
  __shared__ TailShared sh;
  extern __shared__ __align__(16) int dyn[];
  const int K = a.K, b = a.b, V = a.V, kb = K * b;
  int* g = dyn;
  double* lq = reinterpret_cast<double*>(dyn + ((kb + 1) & ~1));
  double* bls = lq + kb;  // lse of branch row (z, i), for the residual's offsets at the draw slot
  double* S = bls + kb;
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const bool report = true;
  DrawCtx& c = sh.c;
  const size_t bbase = static_cast<size_t>(r) * kb;  // component row (r, z, i) = bbase + z * b + i

  // A. header, draft tokens, mixing logits, branch argmax
  const int pb = a.pos_off[r], pe = a.pos_off[r + 1], tb = a.tgt_off[r], te = a.tgt_off[r + 1];
  const float T = a.T[r], Tb = a.branch_T[r];
  const int x0 = a.x[static_cast<size_t>(r) * b + min(tid, b - 1)];
  const float m0 = a.mix[static_cast<size_t>(r) * K + min(tid, K - 1)];
  for (int k = tid; k < kb; k += kSumNT) g[k] = a.barg[bbase + k];
  exp_table_init(sh.etab);
  if (tid < b) sh.x[tid] = x0;
  if (tid < K) sh.mix[tid] = m0;
  __syncthreads();
  const int Lr = pe - pb;
  if (!(Lr >= 0 && Lr <= b && te - tb == Lr + 1)) {
    if (report && tid == 0) {
      raise_status(a.status, SV_ST_BAD_OFFSETS);
      a.n_acc[r] = 0;
      a.rec[r].mode = kDrawNone;
    }
    return;
  }
  const bool greedy = T == 0.0f, softb = Tb > 0.0f;
  const double invT = 1.0 / static_cast<double>(T), Tbd = static_cast<double>(Tb);

  // B. candidate rows' statistics; log q_i(x_i | z) for i < L_r; log q(z | y)
  const int is = min(tid, Lr);
  const float rc0 = a.row_cut[tb + is];
  const double rk0 = a.row_kept[tb + is];
  const int ra0 = a.row_argmax[tb + is];
  if (tid <= Lr) {
    sh.rc[tid] = rc0;
    sh.rk[tid] = rk0;
    sh.ra[tid] = ra0;
  }
  for (int k = tid; k < K * Lr; k += kSumNT) {
    const int z = k / Lr, i = k - z * Lr;
    const int xv = sh.x[i];
    double v = -INFINITY;
    const size_t row = bbase + static_cast<size_t>(z) * b + i;
    const double bl = softb ? a.blse[row] : 0.0;
    if (xv >= 0 && xv < V) {
      if (softb)
        v = static_cast<double>(load_val<DT>(row_ptr(a.comp, DT, static_cast<int64_t>(row), a.comp_ld), xv)) / Tbd -
            bl;
      else
        v = g[z * b + i] == xv ? 0.0 : -INFINITY;
    }
    lq[z * b + i] = v;
    bls[z * b + i] = bl;
  }
  if (wv == 1) {  // log q(z | y), q(z | y) = softmax of the mixing logits
    const bool act = lane < K;
    const float ml = act ? sh.mix[lane] : -INFINITY;
    const float mmax = wave_max_f32(ml);
    const double e = act ? exp(static_cast<double>(ml) - static_cast<double>(mmax)) : 0.0;
    const double lsum = log(wave_sum_f64(e));
    sh.pi[lane] = act ? (static_cast<double>(ml) - static_cast<double>(mmax)) - lsum : -INFINITY;
  }
  const uint64_t seed = *a.seed;
  double p = 0.0, u = 0.0;
  bool xok = true;
  if (tid < kWave) {  // lane i < L_r: p(x_i) and u_i (word 0)
    u = u24(philox_at(seed, static_cast<uint32_t>(lane), static_cast<uint32_t>(r)).x);
    if (lane < Lr) {
      const int xv = sh.x[lane];
      xok = xv >= 0 && xv < V;
      if (xok)
        p = greedy ? (xv == ra0 ? 1.0 : 0.0)
                   : p_of(load_val<DT>(row_ptr(a.tgt, DT, tb + lane, a.tgt_ld), xv), rc0, invT, rk0, sh.etab);
      else if (report)
        raise_status(a.status, SV_ST_BAD_TOKEN);
    }
  }
  __syncthreads();
  // running log posterior, in position order: lane z of wave 0
  if (tid < K) {
    double run = sh.pi[tid];
    S[tid] = run;
    for (int i = 0; i < Lr; ++i) {
      run += lq[tid * b + i];
      S[(i + 1) * K + tid] = run;
    }
  }
  if (report && wv >= 1)  // the branch argmax, i < L_r
    for (int k = tid - kWave; k < kb; k += kSumNT - kWave)
      if (k % b < Lr) a.branch_out[bbase + k] = g[k];
  __syncthreads();

  // C1. the exponentials, one (position, branch) per thread (table method;
  // arguments <= 0): S becomes exp(S_iz - M_i) and lq becomes q_i(x_i | z)
  for (int i = tid; i <= Lr; i += kSumNT) {
    double M = -INFINITY;
    for (int z = 0; z < K; ++z) M = fmax(M, S[i * K + z]);
    sh.mrow[i] = M;
  }
  __syncthreads();
  for (int k = tid; k < (Lr + 1) * K; k += kSumNT) {
    const int i = k / K, z = k - i * K;
    const double M = sh.mrow[i];
    S[k] = M > -INFINITY ? exp_tab(S[k] - M, sh.etab) : 0.0;
    if (i < Lr) {
      const double l = lq[z * b + i];
      lq[z * b + i] = l > -INFINITY ? exp_tab(l, sh.etab) : 0.0;
    }
  }
  __syncthreads();

  // C. acceptance and the draw context (wave 0)
  if (tid < kWave) {
    // lane i: w_z^(i) = exp(S_iz - M) / sum, q(x_i | x_<i) = sum_z w_z q_i(x_i | z)
    const int il = min(lane, Lr);
    const double* Si = S + static_cast<size_t>(il) * K;  // the exponentials of C1
    const double M = sh.mrow[il];
    double tot = 0.0;
    if (M > -INFINITY)
      for (int z = 0; z < K; ++z) tot += Si[z];
    double q = 0.0;
    if (lane < Lr && M > -INFINITY) {
      for (int z = 0; z < K; ++z) {
        const double w = Si[z] / tot;
        if (w != 0.0) q += w * lq[z * b + lane];
      }
    }
    if (lane < Lr && !xok) q = 0.0;
    const bool pos = lane < Lr;
    bool reject = false;
    if (pos) {
      reject = !(q > 0.0 ? u < p / q : p > 0.0);
      if (report) {
        const size_t k = static_cast<size_t>(r) * b + lane;
        if (a.p_out) a.p_out[k] = p;
        if (a.q_out) a.q_out[k] = q;
        if (a.u_out) a.u_out[k] = static_cast<float>(u);
        a.q_at_draft[k] = q;
        double* pw = a.post_w + k * K;
        for (int z = 0; z < K; ++z) pw[z] = M > -INFINITY ? Si[z] / tot : 0.0;
        if (!(M > -INFINITY)) raise_status(a.status, SV_ST_EMPTY_POSTERIOR);
      }
    }
    const uint64_t mask = __ballot(reject);
    const int n = mask ? __ffsll(static_cast<long long>(mask)) - 1 : Lr;
    if (report && lane == 0) a.n_acc[r] = n;
    const bool res = !greedy && n < Lr;
    if (lane == 0) {
      c.n = n;
      c.bonus = n == Lr ? 1 : 0;
      c.mode = greedy ? kDrawGreedy : (n == Lr ? kDrawP : (softb ? kDrawSoft : kDrawResidual));
      c.token = sh.ra[n];
      c.cut = sh.rc[n];
      c.kept = sh.rk[n];
      c.invT = invT;
      c.dlse = 0.0;
      c.invTb = softb ? 1.0 / Tbd : 0.0;
      c.trow = tb + n;
      c.drow = static_cast<int64_t>(bbase) + n;  // branch 0's row at slot n; branch z: + z * b
      c.ncorr = 0;
    }
    if (res && lane == n)  // the posterior at the draw slot, one weight per branch
      for (int z = 0; z < K; ++z) sh.tw[z] = M > -INFINITY ? Si[z] / tot : 0.0;
    __syncwarp();
    if (res) {
      const bool in = lane < K;
      const double w = in ? sh.tw[lane] : 0.0;
      if (softb) {
        const double bl = in ? bls[lane * b + n] : 0.0;  // n < L_r: stored in B
        if (in) c.cw[lane] = w > 0.0 ? bl - log(w) : INFINITY;
        if (lane == 0) c.ncorr = K;
      } else {
        const int v = in ? g[lane * b + n] : -1;
        build_corrections(c, K, in && w > 0.0 && v >= 0 && v < V, v, w);
      }
    }
    __syncwarp();
    if (report) write_record(a, r, c);
  }
}

// The soft tail's sums over the drawn row (one block per (request, chunk)),
// from the draw record of k_soft_head: for a soft residual each wave sums
// kSoftSubs sub-chunks (over the nucleus lists for bf16 rows and K <= kSoftB);
// a p or greedy-branch draw sums the block's chunk as the greedy tail does.
template <int DT>
__global__ __launch_bounds__(kSumNT) void k_soft_body(SampleArgs a) {
  __shared__ DrawCtx c;
  __shared__ double etab[kExpTab];
  extern __shared__ __align__(16) int dyn[];
  const int S4 = soft_chunks(a.V);
  const int r = blockIdx.x / S4, ch = blockIdx.x % S4;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  exp_table_init(etab);
  if (tid < kWave) {
    const DrawRec& d = a.rec[r];
    const int nc = d.ncorr;
    if (lane == 0) {
      c.mode = d.mode; c.n = d.n; c.bonus = d.bonus; c.token = d.token; c.ncorr = nc;
      c.cut = d.cut; c.invT = d.invT; c.kept = d.kept; c.dlse = d.dlse; c.invTb = d.invTb;
      c.trow = d.trow; c.drow = d.drow;
    }
    if (lane < nc) {
      c.ctok[lane] = d.ctok[lane];
      c.cw[lane] = d.cw[lane];
      c.cq[lane] = d.cq[lane];
    }
  }
  __syncthreads();
  if (c.mode == kDrawGreedy || c.mode == kDrawNone) return;
  if (c.mode == kDrawSoft) {
    for (int j = 0; j < kSoftSubs; ++j) {
      const int sub = ch * kSoftChunk + j * (kSumNT / kWave) + wv;
      if (sub >= a.NSUB) break;  // wave-uniform
      if (DT == SV_BF16 && a.K <= kSoftB)
        sub_sum_soft_lists(a, c, r, sub, etab, reinterpret_cast<char*>(dyn));
      else
        sub_sum_soft<DT>(a, c, r, sub, etab);
    }
  } else {
    sub_sums<DT, DT, false>(a, c, r, ch, reinterpret_cast<float*>(dyn), etab);
  }
}

// The draw: one wave per request, after the sums.  Lane l holds the sub-chunk
// sums [l*spt, (l+1)*spt); a wave scan finds the sub-chunk holding t = u * W,
// then the lanes take its 64 groups and a second scan finds the token.
constexpr int kPickCache = 8;  // sub-chunk sums kept in registers per lane

template <int DT, int DDT, bool kDense, bool kSoft>
__global__ __launch_bounds__(kWave) void k_pick(SampleArgs a) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const DrawRec& rec = a.rec[r];
  const int mode = rec.mode, n = rec.n, bonus = rec.bonus, rtok = rec.token, nc = kDense ? 0 : rec.ncorr;
  const int64_t trow = rec.trow, drow = rec.drow;
  const float cut = rec.cut;
  const double invT = rec.invT, kept = rec.kept, dlse = rec.dlse;
  const uint64_t seed = *a.seed;
  const int V = a.V, NSUB = a.NSUB;
  const int spt = (NSUB + kWave - 1) / kWave;
  const int s0 = min(NSUB, lane * spt), s1 = min(NSUB, s0 + spt);
  const double* subp = a.sub + static_cast<size_t>(r) * NSUB * 2;
  // this round's loads (clamped in-bounds) are all issued before any is used
  double cw_[kPickCache], cp_[kPickCache];
#pragma unroll
  for (int k = 0; k < kPickCache; ++k) {
    const int s = min(s0 + k, NSUB - 1);
    cw_[k] = subp[2 * s];
    cp_[k] = subp[2 * s + 1];
  }
  const int ctok = kDense ? -1 : rec.ctok[lane];
  const double cqt = kDense ? 0.0 : rec.cq[lane];
  asm volatile("" ::: "memory");  // every load above is issued before any is used
  __shared__ double etab[kExpTab];
  __shared__ __align__(16) char plists[kSoft ? SoftLists::kPerWave : 16];  // soft residual: the nucleus list
  __shared__ double wsub[kSoft ? kSubG * 8 : 1];                              // and the sub-chunk's weights
  exp_table_init(etab);
  __syncthreads();
  double lw = 0.0, lp = 0.0;
#pragma unroll
  for (int k = 0; k < kPickCache; ++k) {
    if (s0 + k < s1) {
      lw += cw_[k];
      lp += cp_[k];
    } else {
      cw_[k] = 0.0;
      cp_[k] = 0.0;
    }
  }
  for (int s = s0 + kPickCache; s < s1; ++s) {  // more than kPickCache sub-chunks per lane
    lw += subp[2 * s];
    lp += subp[2 * s + 1];
  }
  if (mode == kDrawNone) return;  // malformed offsets (reported by the sums kernel)
  if (mode == kDrawGreedy) {      // p is one-hot at the argmax, and so is the residual
    if (lane == 0) {
      a.token[r] = rtok;
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
  const int NG = groups_of(V);
  const int g = sub * kSubG + lane;
  double w8[8];
  bool formed = false;
  if constexpr (kSoft) {
    if (mode == kDrawSoft && !use_p) {  // the same weights as the sums kernel formed
      const size_t cstride = static_cast<size_t>(a.b) * static_cast<size_t>(a.comp_ld) * (DT == SV_BF16 ? 2 : 4);
      const char* trowp = row_ptr(a.tgt, DT, trow, a.tgt_ld);
      const char* crow0 = row_ptr(a.comp, DT, drow, a.comp_ld);
      if (DT == SV_BF16 && a.K <= kSoftB) {  // over the nucleus only, as the sums kernel did
#pragma unroll
        for (int q = 0; q < 8; ++q) wsub[lane * 8 + q] = 0.0;
        __syncwarp();
        soft_nucleus(a, trowp, crow0, cstride, rec.cw, sub, cut, invT, kept, rec.invTb, etab, plists,
                     [&](int i, double, double w) { wsub[i] = w; });
        __syncwarp();
#pragma unroll
        for (int q = 0; q < 8; ++q) w8[q] = wsub[lane * 8 + q];
      } else {
        double p8[8], s8[8];
        soft_group<DT>(a, trowp, crow0, cstride, rec.cw, g, cut, invT, kept, rec.invTb, etab, p8, s8);
#pragma unroll
        for (int q = 0; q < 8; ++q) w8[q] = s8[q];
      }
      formed = true;
    }
  }
  if (!formed) {
    const int gc = min(g, NG - 1);
    const bool dense_res = kDense && !use_p;
    uint4 t0, t1, d0, d1;
    raw8<DT>(row_ptr(a.tgt, DT, trow, a.tgt_ld), gc, V, t0, t1);
    if (dense_res) raw8<DDT>(row_ptr(a.draft, DDT, drow, a.draft_ld), gc, V, d0, d1);
    float l[8], d[8];
    decode8<DT>(t0, t1, g, V, g < NG, l);
    if (dense_res) decode8<DDT>(d0, d1, g, V, g < NG, d);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      double w = p_of(l[q], cut, invT, kept, etab);  // 0 past V (value -inf) unless the cut is -inf
      if (!(l[q] > -INFINITY)) w = 0.0;
      if (dense_res) {
        const double t2 = w - exp_tab(static_cast<double>(d[q]) * invT - dlse, etab);
        w = t2 > 0.0 ? t2 : 0.0;
      }
      w8[q] = w;
    }
    if (!kDense && !use_p) {  // branch tokens: max(0, p - q)
      for (int t2 = 0; t2 < nc; ++t2) {
        const int v = bcast_i32(ctok, t2);
        const double qv = bcast_f64(cqt, t2);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (v == g * 8 + q) {
            const double d = w8[q] - qv;
            w8[q] = d > 0.0 ? d : 0.0;
          }
      }
    }
  }
  double lsum = 0.0;
#pragma unroll
  for (int q = 0; q < 8; ++q) lsum += w8[q];
  const double inc2 = wave_incl_scan_f64(lsum);
  const uint64_t hit = __ballot(g < NG && base + inc2 > t);
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

// ------------------------------------------------------------------ draws from prepared records
// The sums of a draw whose record (a.rec[r]) an earlier kernel wrote: the
// tree verification's walk.  Dense proposals only (SV_Q_DENSE weights).
template <int DT, int DDT>
__global__ __launch_bounds__(kSumNT) void k_rec_sums(SampleArgs a) {
  __shared__ double etab[kExpTab];
  __shared__ DrawCtx c;
  extern __shared__ __align__(16) int dyn[];
  const int r = blockIdx.x / a.S, ch = blockIdx.x % a.S;
  exp_table_init(etab);
  if (threadIdx.x == 0) {
    const DrawRec& d = a.rec[r];
    c.mode = d.mode; c.n = d.n; c.bonus = d.bonus; c.token = d.token; c.ncorr = 0;
    c.trow = d.trow; c.drow = d.drow; c.cut = d.cut; c.invT = d.invT; c.kept = d.kept; c.dlse = d.dlse;
    c.invTb = 0.0;
  }
  __syncthreads();
  if (c.mode != kDrawResidual && c.mode != kDrawP) return;  // greedy (the pick takes the argmax), or none
  sub_sums<DT, DDT, true>(a, c, r, ch, reinterpret_cast<float*>(dyn), etab);
}

template <int DT, int DDT>
static int32_t launch_record_draw_t(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_rec_sums<DT, DDT>), dim3(a.R * a.S), dim3(kSumNT), DLists<true>::kBytes, s, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((k_pick<DT, DDT, true, false>), dim3(a.R), dim3(kWave), 0, s, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

int32_t launch_record_draw(const SampleArgs& a, hipStream_t s) {
  const bool bf = a.dtype == SV_BF16, dbf = a.ddtype == SV_BF16;
  if (bf) return dbf ? launch_record_draw_t<SV_BF16, SV_BF16>(a, s) : launch_record_draw_t<SV_BF16, SV_F32>(a, s);
  return dbf ? launch_record_draw_t<SV_F32, SV_BF16>(a, s) : launch_record_draw_t<SV_F32, SV_F32>(a, s);
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
template <int DT, int DDT, bool kDense, bool kAccept>
static int32_t launch_draw_t(const SampleArgs& a, hipStream_t s) {
  const size_t kb = static_cast<size_t>(a.K) * a.b;
  const size_t tables = kDense ? 0 : sizeof(int) * ((kb + 1) & ~static_cast<size_t>(1)) + sizeof(double) * kb;
  const size_t dyn = tables > DLists<kDense>::kBytes ? tables : DLists<kDense>::kBytes;
  hipLaunchKernelGGL((k_draw_sums<DT, DDT, kDense, kAccept>), dim3(a.R * a.S), dim3(kSumNT), dyn, s, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((k_pick<DT, DDT, kDense, false>), dim3(a.R), dim3(kWave), 0, s, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

// soft branches: the soft tail, then the pick
template <int DT>
static int32_t launch_draw_soft(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_soft_head<DT>), dim3(a.R), dim3(kSumNT), soft_tables_bytes(a.K, a.b), s, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  size_t dyn = DLists<false>::kBytes;
  if (DT == SV_BF16 && a.K <= kSoftB && SoftLists::kBytes > dyn) dyn = SoftLists::kBytes;
  hipLaunchKernelGGL((k_soft_body<DT>), dim3(a.R * soft_chunks(a.V)), dim3(kSumNT), dyn, s, a);
  if (hipGetLastError() != hipSuccess) return SV_ERR_LAUNCH;
  hipLaunchKernelGGL((k_pick<DT, DT, false, true>), dim3(a.R), dim3(kWave), 0, s, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

template <bool kAccept>
static int32_t launch_draw(const SampleArgs& a, hipStream_t s) {
  const bool bf = a.dtype == SV_BF16, dbf = a.ddtype == SV_BF16;
  if (a.q_mode == SV_Q_MIXTURE)
    return bf ? launch_draw_t<SV_BF16, SV_BF16, false, kAccept>(a, s) : launch_draw_t<SV_F32, SV_F32, false, kAccept>(a, s);
  if (bf)
    return dbf ? launch_draw_t<SV_BF16, SV_BF16, true, kAccept>(a, s) : launch_draw_t<SV_BF16, SV_F32, true, kAccept>(a, s);
  return dbf ? launch_draw_t<SV_F32, SV_BF16, true, kAccept>(a, s) : launch_draw_t<SV_F32, SV_F32, true, kAccept>(a, s);
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
  return launch_draw<false>(a, static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------ allocation-free draw
// sv_residual_sample_noalloc keeps the draw records and sub-chunk sums in this
// file-scope array instead of a caller workspace.  Host code never passes the
// array's name to a kernel: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept in g_scratch_dev.
// Nothing in it must start at zero: every call rewrites each record it uses and
// every sub-chunk sum its pick reads.  Calls that overlap on one GPU share it
// and race.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_dev[dev] = ptr;
  }
  return g_scratch_dev[dev];
}
}  // namespace

extern "C" int32_t sv_residual_sample_noalloc(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                              const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                                              const float* temperature, const int32_t* row_argmax,
                                              const float* row_cut, const double* row_kept_lse, int32_t q_mode,
                                              const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                                              const int32_t* draft_argmax, const double* draft_lse, int32_t K,
                                              const int32_t* branch_tok, const double* post_w, const uint64_t* seed,
                                              const int32_t* n_acc, int32_t* token, int32_t* is_bonus,
                                              uint32_t* status, void* stream) {
  if (!sample_args_ok(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                      row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed, status))
    return SV_ERR_ARG;
  if (!n_acc || !token || !is_bonus) return SV_ERR_ARG;
  if (q_mode == SV_Q_MIXTURE && (K < 1 || K > 64 || !branch_tok || !post_w)) return SV_ERR_ARG;
  const size_t rec_bytes = align256(sizeof(DrawRec) * static_cast<size_t>(R));
  const size_t sub_bytes = sizeof(double) * 2 * static_cast<size_t>(R) * static_cast<size_t>(sub_chunks(V));
  if (rec_bytes + sub_bytes > SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_TOO_LARGE;
  void* ptr = scratch_on_current_device();
  if (!ptr) return SV_ERR_LAUNCH;
  SampleArgs a = sample_args(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                             row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed,
                             ptr);
  a.status = status;
  a.rec = reinterpret_cast<DrawRec*>(ptr);
  a.sub = reinterpret_cast<double*>(static_cast<char*>(ptr) + rec_bytes);
  a.K = q_mode == SV_Q_MIXTURE ? K : 0; a.branch_tok = branch_tok; a.post_w = const_cast<double*>(post_w);
  a.n_acc_in = n_acc; a.token = token; a.is_bonus = is_bonus;
  return launch_draw<false>(a, static_cast<hipStream_t>(stream));
}

extern "C" int32_t sv_accept_sample(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                    const int32_t* tgt_off, const int32_t* pos_off, int32_t R, int32_t b,
                                    const float* temperature, const int32_t* row_argmax, const float* row_cut,
                                    const double* row_kept_lse, const int32_t* draft_tok, int32_t q_mode,
                                    const void* draft_logits, int32_t draft_dtype, int64_t draft_ld,
                                    const int32_t* draft_argmax, const double* draft_lse, int32_t K,
                                    const float* mix_logits, const void* comp_logits, int64_t comp_ld,
                                    const float* branch_T, int32_t* branch_tok, double* post_w,
                                    double* q_at_draft, const uint64_t* seed, int32_t* n_acc, int32_t* token,
                                    int32_t* is_bonus, double* p_out, double* q_out, float* u_out, void* ws,
                                    size_t ws_bytes, void* stream) {
  if (!sample_args_ok(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                      row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed, ws))
    return SV_ERR_ARG;
  if (!draft_tok || !n_acc || !token || !is_bonus) return SV_ERR_ARG;
  if (q_mode == SV_Q_MIXTURE && (K < 1 || K > 64 || !mix_logits || !branch_tok || !post_w || !q_at_draft))
    return SV_ERR_ARG;
  const bool soft = branch_T != nullptr;
  if (soft) {
    if (q_mode != SV_Q_MIXTURE || !comp_logits || comp_ld < V || !rows_aligned(comp_logits, dtype, comp_ld))
      return SV_ERR_ARG;
    if (static_cast<long long>(K) * b > kSoftMaxKb) return SV_ERR_ARG;
  }
  const WsLayout l = ws_layout(R, b, q_mode == SV_Q_MIXTURE ? K : 0, V);
  if (ws_bytes < l.total) return SV_ERR_WORKSPACE;
  SampleArgs a = sample_args(tgt_logits, dtype, tgt_ld, V, tgt_off, pos_off, R, b, temperature, row_argmax, row_cut,
                             row_kept_lse, q_mode, draft_logits, draft_dtype, draft_ld, draft_argmax, draft_lse, seed,
                             ws);
  a.x = draft_tok; a.K = q_mode == SV_Q_MIXTURE ? K : 0; a.mix = mix_logits; a.branch_out = branch_tok;
  a.bkey = reinterpret_cast<const uint64_t*>(static_cast<char*>(ws) + l.bkey);
  a.slot = reinterpret_cast<const SlotRec*>(static_cast<char*>(ws) + l.slot);
  a.dslot = reinterpret_cast<const SlotRec*>(static_cast<char*>(ws) + l.dslot);
  a.post_w = post_w; a.q_at_draft = q_at_draft; a.n_acc = n_acc; a.n_acc_in = n_acc; a.token = token;
  a.is_bonus = is_bonus; a.p_out = p_out; a.q_out = q_out; a.u_out = u_out;
  if (soft) {
    a.comp = comp_logits; a.comp_ld = comp_ld; a.branch_T = branch_T;
    a.blse = reinterpret_cast<const double*>(static_cast<char*>(ws) + l.blse);
    a.barg = reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + l.barg);
    hipStream_t st = static_cast<hipStream_t>(stream);
    return dtype == SV_BF16 ? launch_draw_soft<SV_BF16>(a, st) : launch_draw_soft<SV_F32>(a, st);
  }
  return launch_draw<true>(a, static_cast<hipStream_t>(stream));
}
