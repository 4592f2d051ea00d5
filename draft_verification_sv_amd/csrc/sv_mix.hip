// sv_mix.hip -- latent-mixture proposal with greedy branches.
//
// "Pith review of DBLAST", "What carries the argument": the block proposal is
// q_dep(x_1:b | y) = sum_z q(z|y) prod_i q_i(x_i | y, z); at inference a
// category is sampled and its branch decoded greedily, and verification
// conditions on the accepted prefix through the category posterior (the
// greedy-branch conditional, Eq. (20) per the Referee report, minor 5).  With
// point-mass branches at g_i(z) = argmax_v c_{r,z,i,v}, the posterior before
// position i keeps the categories whose branch agrees with the draft prefix:
//   w_z = q(z|y) [g_j(z) = x_j, j < i] / sum over z of the same,
//   q(x_i | x_<i) = sum of w_z over z with g_i(z) = x_i.
//
// Work split: the K * L_r component rows of every request are cut into S
// chunks; one 256-thread block streams one chunk with 128-bit loads and
// reduces (max value, lowest index) in registers, then in the wave and the
// block.  Each block stores its chunk result and counts in on the request's
// counter; the last block of a request merges the chunk results in fixed order
// and runs the posterior recursion over the positions with one lane per
// category (K <= 64), in double.
#include <math.h>

#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

constexpr int kMixNT = 256;

struct MixArgs {
  const void* comp;
  int64_t ld;
  int V, K, b;
  const float* mix;
  const int32_t* pos_off;
  int R, max_pos;
  const int32_t* x;
  int32_t* branch_tok;
  double* post_w;
  double* q;
  uint32_t* counters;  // [R]
  uint64_t* part;      // [max_pos * K * S]
  int S;               // chunks per row
  int CV;              // 16-byte vectors per chunk
  uint32_t* status;
};

// Order-preserving key of a float with -0 folded onto +0.
__device__ __forceinline__ uint32_t fkey(float f) {
  f = f + 0.0f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float max8(float a0, float a1, float a2, float a3, float a4, float a5, float a6, float a7) {
  return fmaxf(fmaxf(fmaxf(a0, a1), fmaxf(a2, a3)), fmaxf(fmaxf(a4, a5), fmaxf(a6, a7)));
}

template <int DT>
__global__ __launch_bounds__(kMixNT) void k_mixture(MixArgs a) {
  __shared__ uint64_t red[kMixNT / kWave];
  __shared__ int s_req;
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const int c = blk % a.S;
  const int z = (blk / a.S) % a.K;
  const int p = blk / (a.S * a.K);
  const int total = a.pos_off[a.R];
  if (blk == 0 && tid == 0 && (a.pos_off[0] != 0 || total > a.max_pos || total < 0))
    raise_status(a.status, SV_ST_BAD_OFFSETS);
  if (p >= total) return;
  const int r = find_request<kMixNT>(a.pos_off, a.R, p, &s_req);
  if (r < 0) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  const int i = p - a.pos_off[r];
  const int Lr = a.pos_off[r + 1] - a.pos_off[r];
  if (Lr > a.b) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  const int64_t row = (static_cast<int64_t>(r) * a.K + z) * a.b + i;
  constexpr int PER = DT == SV_BF16 ? 8 : 4;  // elements per 16-byte vector
  const size_t esz = DT == SV_BF16 ? 2 : 4;
  const char* rowp = static_cast<const char*>(a.comp) + static_cast<size_t>(row) * static_cast<size_t>(a.ld) * esz;
  const uint4* vp = reinterpret_cast<const uint4*>(rowp);
  const int nvec = a.V / PER;
  const int v0 = c * a.CV;
  const int v1 = min(nvec, v0 + a.CV);

  float best = -INFINITY;
  int bvi = -1;
  uint4 bv = {0, 0, 0, 0};
  auto vmax = [](const uint4& d) -> float {
    if constexpr (DT == SV_BF16) {
      return max8(bf16_lo(d.x), bf16_hi(d.x), bf16_lo(d.y), bf16_hi(d.y), bf16_lo(d.z), bf16_hi(d.z), bf16_lo(d.w),
                  bf16_hi(d.w));
    } else {
      return fmaxf(fmaxf(__uint_as_float(d.x), __uint_as_float(d.y)), fmaxf(__uint_as_float(d.z), __uint_as_float(d.w)));
    }
  };
  int v = v0 + tid;
  for (; v + 3 * kMixNT < v1; v += 4 * kMixNT) {
    const uint4 d0 = load16_stream(vp + v);
    const uint4 d1 = load16_stream(vp + v + kMixNT);
    const uint4 d2 = load16_stream(vp + v + 2 * kMixNT);
    const uint4 d3 = load16_stream(vp + v + 3 * kMixNT);
    float m;
    m = vmax(d0);
    if (m > best) { best = m; bvi = v; bv = d0; }
    m = vmax(d1);
    if (m > best) { best = m; bvi = v + kMixNT; bv = d1; }
    m = vmax(d2);
    if (m > best) { best = m; bvi = v + 2 * kMixNT; bv = d2; }
    m = vmax(d3);
    if (m > best) { best = m; bvi = v + 3 * kMixNT; bv = d3; }
  }
  for (; v < v1; v += kMixNT) {
    const uint4 d0 = load16_stream(vp + v);
    const float m = vmax(d0);
    if (m > best) { best = m; bvi = v; bv = d0; }
  }
  int bidx = -1;
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
  if (c == a.S - 1) {  // elements past the last full vector
    const int e = nvec * PER + tid;
    if (e < a.V) {
      const float f = load_val<DT>(rowp, e);
      if (f > best || bidx < 0) {
        best = f;
        bidx = e;
      }
    }
  }
  uint64_t packed = bidx >= 0 ? (static_cast<uint64_t>(fkey(best)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bidx)) : 0;
  packed = block_max_u64<kMixNT>(packed, red);
  if (tid == 0) {
    a.part[(static_cast<size_t>(p) * a.K + z) * a.S + c] = packed;
    s_last = arrive_last(&a.counters[r], static_cast<uint32_t>(Lr) * a.K * a.S) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid >= kWave) return;

  // ---- last block of request r: branch tokens and the posterior recursion
  const int lane = tid;
  const bool act = lane < a.K;
  const float ml = act ? a.mix[static_cast<size_t>(r) * a.K + lane] : -INFINITY;
  float mmax = ml;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, o, kWave));
  const double e = act ? exp(static_cast<double>(ml) - static_cast<double>(mmax)) : 0.0;
  const double pi = e / wave_sum_f64(e);  // q(z | y)
  bool consistent = act;
  const int base = a.pos_off[r];
  for (int ii = 0; ii < Lr; ++ii) {
    int g = 0;
    if (act) {
      uint64_t best_p = 0;
      const uint64_t* pp = a.part + (static_cast<size_t>(base + ii) * a.K + lane) * a.S;
      for (int cc = 0; cc < a.S; ++cc) {
        const uint64_t t = load_acquire_relaxed(pp + cc);
        best_p = t > best_p ? t : best_p;
      }
      g = best_p ? static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best_p)) : 0;
      a.branch_tok[(static_cast<size_t>(r) * a.K + lane) * a.b + ii] = g;
    }
    const double w = consistent ? pi : 0.0;
    const double sw = wave_sum_f64(w);
    const double post = sw > 0.0 ? w / sw : 0.0;
    if (act) a.post_w[(static_cast<size_t>(r) * a.b + ii) * a.K + lane] = post;
    const int xi = a.x[static_cast<size_t>(r) * a.b + ii];
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

extern "C" int32_t sv_mixture_q(const void* comp_logits, int32_t dtype, int64_t ld, int32_t V, int32_t K, int32_t b,
                                const float* mix_logits, const int32_t* pos_off, int32_t R, int32_t max_pos,
                                const int32_t* draft_tok, int32_t* branch_tok, double* post_w, double* q_at_draft,
                                void* ws, size_t ws_bytes, void* stream) {
  if (!comp_logits || !mix_logits || !pos_off || !draft_tok || !branch_tok || !post_w || !q_at_draft || !ws)
    return SV_ERR_ARG;
  if (R < 1 || V < 1 || K < 1 || K > 64 || b < 1 || b > 64 || ld < V || max_pos < 0) return SV_ERR_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_ARG;
  if (!rows_aligned(comp_logits, dtype, ld)) return SV_ERR_ARG;
  if (max_pos > R * b) return SV_ERR_ARG;
  const WsLayout l = ws_layout(R, b, K, V);
  if (ws_bytes < l.total) return SV_ERR_WORKSPACE;
  if (max_pos == 0) return SV_OK;
  const int per = dtype == SV_BF16 ? 8 : 4;
  const int nvec = V / per;
  const int S = mix_chunks(V, dtype);
  int CV = (nvec + S - 1) / S;
  if (CV < 1) CV = 1;
  MixArgs a{comp_logits, ld, V, K, b, mix_logits, pos_off, R, max_pos, draft_tok, branch_tok, post_w, q_at_draft,
            counters(ws, l.counters), reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + l.mix_part), S, CV,
            status_word(ws)};
  const long long grid = static_cast<long long>(max_pos) * K * S;
  if (grid > 0x7FFFFFFFLL) return SV_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(k_mixture<SV_BF16>, dim3(static_cast<unsigned>(grid)), dim3(kMixNT), 0, s, a);
  else
    hipLaunchKernelGGL(k_mixture<SV_F32>, dim3(static_cast<unsigned>(grid)), dim3(kMixNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
