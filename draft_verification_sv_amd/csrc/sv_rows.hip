// sv_rows.hip -- per-row target/draft statistics: maximum, argmax, log-sum-exp
// at temperature T and the top-p (nucleus) cut.
//
// Sampling filter: temperature softmax with top-p ("Pith review of DBLAST",
// "What would settle it": target sampling at T = 1.5, top-p 0.95; nucleus
// sampling is its reference [18]).
//
// bf16 rows, one pass over HBM.  A bf16 logit takes one of 65536 values and
// every token with the same value has the same probability, so the exact count
// of tokens per value determines the maximum, sum_v exp(l_v/T) and the top-p cut
// (the first value, from the top, at which the cumulative mass reaches top_p).
// The counts go into an LDS histogram indexed by value for all |l| in
// [2^-24, 2^24) (48 binades x 128 mantissas per sign = 12288 bins, 48 KiB as
// u32).  Integer counts are exact and order-independent, so the result is
// deterministic.  The masses count * exp(v/T - m/T) are then formed once per
// non-empty bin in double.  Rows holding a value outside that range (zero,
// |l| < 2^-24, |l| >= 2^24, NaN, Inf) take the generic path below instead.
//
// Generic path (fp32 rows, or bf16 rows outside the histogram range): max and
// argmax, then sum exp(l/T - m/T) in double, then the cut by bisection over
// the monotone 32-bit key of the values (at most 32 passes over the row, which
// stays in cache).  Exact, slow; fp32 rows appear only in small problems.
#include <math.h>

#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

constexpr int kRowNT = 1024;
constexpr int kRowBatch = 8;  // 16-byte loads in flight per thread (double-buffered)
constexpr uint32_t kExpLo = 103u << 7;  // |v| >= 2^-24: biased exponent 103
constexpr int kSide = 6144;             // 48 exponents x 128 mantissas
constexpr int kNBins = 2 * kSide + 2;   // [0] negative special, [1..6144] negative values,
                                        // [6145..12288] positive values, [12289] positive special
constexpr int kBinsPerThread = 2 * kSide / kRowNT;
static_assert(kBinsPerThread * kRowNT == 2 * kSide, "bins must split evenly over the block");

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

// Histogram bins of the two bf16 values packed in w (low half = lower index).
// Bins ascend with the value; out-of-range magnitudes land in the two special
// bins 0 (negative) and 12289 (positive).
__host__ __device__ inline uint32_t bins_of_pair(uint32_t w) {
  const u16x2 h = __builtin_bit_cast(u16x2, w);
  const u16x2 mag = h & (u16x2)(0x7FFF);
  const u16x2 t = mag - (u16x2)(kExpLo);  // wraps to large values below the range
  const u16x2 tc = __builtin_elementwise_min(t, (u16x2)(kSide));
  const u16x2 neg = __builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, h) >> 15);  // 0xFFFF if negative
  const u16x2 bin = (tc ^ neg) + (u16x2)(kSide + 1);  // negative: 6144 - tc, positive: 6145 + tc
  return __builtin_bit_cast(uint32_t, bin);
}

__host__ __device__ inline uint32_t bin_of(uint32_t h16) { return bins_of_pair(h16) & 0xFFFFu; }

// Exact value of an in-range bin (1..12288).
__host__ __device__ inline float bin_value(int bin) {
  uint32_t h;
  if (bin <= kSide)
    h = 0x8000u | static_cast<uint32_t>(kSide - bin + static_cast<int>(kExpLo));
  else
    h = static_cast<uint32_t>(bin - (kSide + 1) + static_cast<int>(kExpLo));
  uint32_t bits = h << 16;
  float f;
  __builtin_memcpy(&f, &bits, 4);
  return f;
}

// Order-preserving 32-bit key of a float (-0 folded onto +0 so equal values share a key).
__host__ __device__ inline uint32_t mono_key(float f) {
  f = f + 0.0f;
  uint32_t b;
  __builtin_memcpy(&b, &f, 4);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__host__ __device__ inline float key_value(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  float f;
  __builtin_memcpy(&f, &b, 4);
  return f;
}

struct RowArgs {
  const void* logits;
  int64_t ld;
  int V;
  const int32_t* row_off;
  int row_stride;
  int R;
  int max_rows;
  const float* T;
  const float* top_p;  // NULL: filter off
  float* row_max;
  int32_t* row_argmax;
  double* row_lse;
  float* row_cut;       // NULL when only statistics are wanted
  double* row_kept_lse;  // NULL when only statistics are wanted
  uint32_t* status;
};

struct RowShared {
  uint64_t red_u64[kRowNT / kWave];
  double red_f64[kRowNT / kWave];
  int red_i32[kRowNT / kWave];
  int req;
  double F;
};

__device__ inline void write_row(const RowArgs& a, int p, float mx, int am, double lse, float cut,
                                 double kept) {
  a.row_max[p] = mx;
  a.row_argmax[p] = am;
  a.row_lse[p] = lse;
  if (a.row_cut) a.row_cut[p] = cut;
  if (a.row_kept_lse) a.row_kept_lse[p] = kept;
}

// ------------------------------------------------------------------ generic path
template <int DT>
__device__ void row_generic(const RowArgs& a, const void* rowp, int p, float T, float tp, bool topp_on,
                            RowShared& sh) {
  const int tid = threadIdx.x;
  const int V = a.V;
  float best = -INFINITY;
  int bidx = -1;
  bool nonfinite = false;
  for (int v = tid; v < V; v += kRowNT) {
    const float f = load_val<DT>(rowp, v);
    nonfinite |= !isfinite(f);
    if (f > best) {
      best = f;
      bidx = v;
    }
  }
  if (nonfinite) raise_status(a.status, SV_ST_NONFINITE);
  uint64_t packed = bidx >= 0 ? (static_cast<uint64_t>(mono_key(best)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bidx)) : 0;
  packed = block_max_u64<kRowNT>(packed, sh.red_u64);
  const float m = packed ? key_value(static_cast<uint32_t>(packed >> 32)) : -INFINITY;
  const int am = packed ? static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(packed)) : 0;
  if (T == 0.0f) {
    if (tid == 0) write_row(a, p, m, am, 0.0, m, 0.0);
    return;
  }
  const double Td = static_cast<double>(T);
  const double M = static_cast<double>(m) / Td;
  double part = 0.0;
  for (int v = tid; v < V; v += kRowNT) part += exp(static_cast<double>(load_val<DT>(rowp, v)) / Td - M);
  const double Z = block_sum_f64<kRowNT>(part, sh.red_f64);
  const double lse = M + log(Z);
  if (!topp_on) {
    if (tid == 0) write_row(a, p, m, am, lse, -INFINITY, lse);
    return;
  }
  const double target = static_cast<double>(tp) * Z;
  // largest key k with F(k) = sum_{key(l) >= k} exp(l/T - M) >= target
  uint64_t lo = 0, hi = static_cast<uint64_t>(mono_key(m)) + 1;
  double F_lo = Z;
  while (hi - lo > 1) {
    const uint64_t mid = (lo + hi) >> 1;
    double s = 0.0;
    for (int v = tid; v < V; v += kRowNT) {
      const float f = load_val<DT>(rowp, v);
      if (mono_key(f) >= mid) s += exp(static_cast<double>(f) / Td - M);
    }
    const double F = block_sum_f64<kRowNT>(s, sh.red_f64);
    if (F >= target) {
      lo = mid;
      F_lo = F;
    } else {
      hi = mid;
    }
  }
  if (tid == 0) write_row(a, p, m, am, lse, key_value(static_cast<uint32_t>(lo)), M + log(F_lo));
}

// ------------------------------------------------------------------ bf16 one-pass path
__device__ __forceinline__ void count_vec(uint32_t* hist, const uint4& d, uint4& bb, uint32_t& vmax) {
  bb.x = bins_of_pair(d.x);
  bb.y = bins_of_pair(d.y);
  bb.z = bins_of_pair(d.z);
  bb.w = bins_of_pair(d.w);
  atomicAdd(&hist[bb.x & 0xFFFFu], 1u);
  atomicAdd(&hist[bb.x >> 16], 1u);
  atomicAdd(&hist[bb.y & 0xFFFFu], 1u);
  atomicAdd(&hist[bb.y >> 16], 1u);
  atomicAdd(&hist[bb.z & 0xFFFFu], 1u);
  atomicAdd(&hist[bb.z >> 16], 1u);
  atomicAdd(&hist[bb.w & 0xFFFFu], 1u);
  atomicAdd(&hist[bb.w >> 16], 1u);
  const u16x2 m2 = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, bb.x), __builtin_bit_cast(u16x2, bb.y)),
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, bb.z), __builtin_bit_cast(u16x2, bb.w)));
  vmax = m2.x > m2.y ? m2.x : m2.y;
}

template <int DT>
__global__ __launch_bounds__(kRowNT) void k_row_stats(RowArgs a) {
  __shared__ RowShared sh;
  __shared__ uint32_t hist[DT == SV_BF16 ? kNBins : 1];
  const int tid = threadIdx.x;
  const int p = blockIdx.x;
  const int total = a.row_off[a.R];
  if (p == 0 && tid == 0 && (a.row_off[0] != 0 || total > a.max_rows || total < 0))
    raise_status(a.status, SV_ST_BAD_OFFSETS);
  if (p >= total) return;
  const int r = find_request<kRowNT>(a.row_off, a.R, p, &sh.req);
  if (r < 0) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  const int j = p - a.row_off[r];
  if (a.row_stride > 0 && j >= a.row_stride) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return;
  }
  const int64_t row = a.row_stride > 0 ? static_cast<int64_t>(r) * a.row_stride + j : static_cast<int64_t>(p);
  const size_t esz = DT == SV_BF16 ? 2 : 4;
  const void* rowp = static_cast<const char*>(a.logits) + static_cast<size_t>(row) * static_cast<size_t>(a.ld) * esz;
  const float T = a.T[r];
  float tp = a.top_p ? a.top_p[r] : 1.0f;
  if (tid == 0 && !(T >= 0.0f)) raise_status(a.status, SV_ST_BAD_TEMPERATURE);
  const bool want_cut = a.row_cut != nullptr;
  bool topp_on = want_cut && a.top_p != nullptr && !(tp >= 1.0f);
  if (topp_on && !(tp > 0.0f)) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_TOP_P);
    tp = 1e-30f;  // keeps the top value only
  }

  if constexpr (DT == SV_BF16) {
    for (int k = tid; k < kNBins; k += kRowNT) hist[k] = 0u;
    __syncthreads();
    const uint16_t* rp = static_cast<const uint16_t*>(rowp);
    const uint4* vp = reinterpret_cast<const uint4*>(rp);
    const int nvec = a.V >> 3;
    uint32_t best = 0;
    int bvec = -1;
    uint4 bbins = {0, 0, 0, 0};
    int v = tid;
    uint4 cur[kRowBatch];
#pragma unroll
    for (int k = 0; k < kRowBatch; ++k)
      if (v + k * kRowNT < nvec) cur[k] = load16_stream(vp + v + k * kRowNT);
    while (v < nvec) {
      const int vn = v + kRowBatch * kRowNT;
      uint4 nxt[kRowBatch];
#pragma unroll
      for (int k = 0; k < kRowBatch; ++k)
        if (vn + k * kRowNT < nvec) nxt[k] = load16_stream(vp + vn + k * kRowNT);
#pragma unroll
      for (int k = 0; k < kRowBatch; ++k) {
        if (v + k * kRowNT < nvec) {
          uint4 bb;
          uint32_t vm;
          count_vec(hist, cur[k], bb, vm);
          if (vm > best) {
            best = vm;
            bvec = v + k * kRowNT;
            bbins = bb;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kRowBatch; ++k) cur[k] = nxt[k];
      v = vn;
    }
    int bidx = -1;
    if (bvec >= 0) {
      const uint32_t h[8] = {bbins.x & 0xFFFFu, bbins.x >> 16, bbins.y & 0xFFFFu, bbins.y >> 16,
                             bbins.z & 0xFFFFu, bbins.z >> 16, bbins.w & 0xFFFFu, bbins.w >> 16};
      int k = 7;
#pragma unroll
      for (int q = 7; q >= 0; --q)
        if (h[q] == best) k = q;
      bidx = bvec * 8 + k;
    }
    const int t0 = nvec << 3;
    if (t0 + tid < a.V) {
      const uint32_t bn = bin_of(rp[t0 + tid]);
      atomicAdd(&hist[bn], 1u);
      if (bn > best || bidx < 0) {
        best = bn;
        bidx = t0 + tid;
      }
    }
    uint64_t packed = bidx >= 0 ? (static_cast<uint64_t>(best) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bidx)) : 0;
    packed = block_max_u64<kRowNT>(packed, sh.red_u64);  // also orders the histogram writes
    const uint32_t special = hist[0] + hist[kNBins - 1];
    if (special == 0u) {
      const int mbin = static_cast<int>(packed >> 32);
      const int am = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(packed));
      const float m = bin_value(mbin);
      if (T == 0.0f) {
        if (tid == 0) write_row(a, p, m, am, 0.0, m, 0.0);
        return;
      }
      const double Td = static_cast<double>(T);
      const double M = static_cast<double>(m) / Td;
      // bins in descending value order: d = 0 is bin 12288
      const int d0 = tid * kBinsPerThread;
      double part = 0.0;
      int last_nonempty = -1;
      for (int k = 0; k < kBinsPerThread; ++k) {
        const int bin = 2 * kSide - (d0 + k);
        const uint32_t c = hist[bin];
        if (c) {
          part += static_cast<double>(c) * exp(static_cast<double>(bin_value(bin)) / Td - M);
          last_nonempty = d0 + k;
        }
      }
      double Z;
      const double prefix = block_excl_scan_f64<kRowNT>(part, sh.red_f64, &Z);
      const double lse = M + log(Z);
      if (!topp_on) {
        if (tid == 0) write_row(a, p, m, am, lse, -INFINITY, lse);
        return;
      }
      const double target = static_cast<double>(tp) * Z;
      int found = 0x7FFFFFFF;
      double Ff = 0.0;
      if (prefix < target) {
        double run = prefix;
        for (int k = 0; k < kBinsPerThread; ++k) {
          const int bin = 2 * kSide - (d0 + k);
          const uint32_t c = hist[bin];
          if (!c) continue;
          run += static_cast<double>(c) * exp(static_cast<double>(bin_value(bin)) / Td - M);
          if (run >= target) {
            found = d0 + k;
            Ff = run;
            break;
          }
        }
      }
      const int dstar = block_min_i32<kRowNT>(found, sh.red_i32);
      if (dstar != 0x7FFFFFFF) {
        if (found == dstar) sh.F = Ff;
        __syncthreads();
        if (tid == 0) write_row(a, p, m, am, lse, bin_value(2 * kSide - dstar), M + log(sh.F));
      } else {
        // rounding kept the cumulative mass below target: keep every token
        const int dlow = -block_min_i32<kRowNT>(-last_nonempty, sh.red_i32);
        if (tid == 0) write_row(a, p, m, am, lse, bin_value(2 * kSide - dlow), lse);
      }
      return;
    }
    // a value outside the histogram range: exact generic path on this row
    row_generic<SV_BF16>(a, rowp, p, T, tp, topp_on, sh);
  } else {
    row_generic<SV_F32>(a, rowp, p, T, tp, topp_on, sh);
  }
}

}  // namespace sv

using namespace sv;

static int32_t launch_rows(const void* logits, int32_t dtype, int64_t ld, int32_t V, const int32_t* row_off,
                           int32_t row_stride, int32_t R, int32_t max_rows, const float* temperature,
                           const float* top_p, float* row_max, int32_t* row_argmax, double* row_lse,
                           float* row_cut, double* row_kept_lse, void* ws, size_t ws_bytes, void* stream) {
  if (!logits || !row_off || !temperature || !row_max || !row_argmax || !row_lse || !ws) return SV_ERR_ARG;
  if (R < 1 || V < 1 || max_rows < 0 || row_stride < 0 || ld < V) return SV_ERR_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_ARG;
  if (!rows_aligned(logits, dtype, ld)) return SV_ERR_ARG;
  if (ws_bytes < 256) return SV_ERR_WORKSPACE;
  if (max_rows == 0) return SV_OK;
  RowArgs a{logits, ld, V, row_off, row_stride, R, max_rows, temperature, top_p, row_max, row_argmax, row_lse,
            row_cut, row_kept_lse, status_word(ws)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == SV_BF16)
    hipLaunchKernelGGL(k_row_stats<SV_BF16>, dim3(max_rows), dim3(kRowNT), 0, s, a);
  else
    hipLaunchKernelGGL(k_row_stats<SV_F32>, dim3(max_rows), dim3(kRowNT), 0, s, a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_softmax_stats(const void* logits, int32_t dtype, int64_t ld, int32_t V,
                                    const int32_t* row_off, int32_t row_stride, int32_t R, int32_t max_rows,
                                    const float* temperature, float* row_max, int32_t* row_argmax,
                                    double* row_lse, void* ws, size_t ws_bytes, void* stream) {
  return launch_rows(logits, dtype, ld, V, row_off, row_stride, R, max_rows, temperature, nullptr, row_max,
                     row_argmax, row_lse, nullptr, nullptr, ws, ws_bytes, stream);
}

extern "C" int32_t sv_topp_threshold(const void* logits, int32_t dtype, int64_t ld, int32_t V,
                                     const int32_t* row_off, int32_t row_stride, int32_t R, int32_t max_rows,
                                     const float* temperature, const float* top_p, float* row_max,
                                     int32_t* row_argmax, double* row_lse, float* row_cut,
                                     double* row_kept_lse, void* ws, size_t ws_bytes, void* stream) {
  if (!row_cut || !row_kept_lse) return SV_ERR_ARG;
  return launch_rows(logits, dtype, ld, V, row_off, row_stride, R, max_rows, temperature, top_p, row_max,
                     row_argmax, row_lse, row_cut, row_kept_lse, ws, ws_bytes, stream);
}

// Host-side self-check of the pure helpers above (runs on the CPU, no GPU).
extern "C" int32_t sv_selftest_rows_host(void) {
  // every in-range bf16 value maps to a bin whose value decodes back to it, and
  // bins ascend with the value
  float prev = -INFINITY;
  for (int bin = 1; bin <= 2 * kSide; ++bin) {
    const float v = bin_value(bin);
    if (!(v > prev)) return 1;
    prev = v;
    uint32_t bits;
    __builtin_memcpy(&bits, &v, 4);
    if (bin_of(bits >> 16) != static_cast<uint32_t>(bin)) return 2;
  }
  for (uint32_t h = 0; h < 65536; ++h) {
    const uint32_t bn = bin_of(h);
    const uint32_t mag = h & 0x7FFFu;
    const bool in = mag >= kExpLo && mag < kExpLo + kSide;
    if (in != (bn >= 1 && bn <= 2u * kSide)) return 3;
    if (!in && bn != ((h & 0x8000u) ? 0u : static_cast<uint32_t>(kNBins - 1))) return 4;
  }
  // pairs: the high half is the second element
  if (bins_of_pair(0x3F80BF80u) != ((bin_of(0x3F80u) << 16) | bin_of(0xBF80u))) return 5;
  // mono_key orders floats, folds -0 onto +0 and inverts
  const float probe[] = {-INFINITY, -1e30f, -2.5f, -1e-30f, -0.0f, 0.0f, 1e-30f, 3.0f, 1e30f, INFINITY};
  for (int k = 0; k + 1 < 10; ++k) {
    if (probe[k] == probe[k + 1]) {
      if (mono_key(probe[k]) != mono_key(probe[k + 1])) return 6;
    } else if (!(mono_key(probe[k]) < mono_key(probe[k + 1]))) {
      return 7;
    }
    if (key_value(mono_key(probe[k])) != probe[k]) return 8;
  }
  return 0;
}
