// sv_rows_dev.hpp -- block-level device code for per-row statistics: maximum,
// argmax, log-sum-exp at temperature T and the top-p (nucleus) cut.
//
// Sampling filter: temperature softmax with top-p ("Pith review of DBLAST",
// "What would settle it": target sampling at T = 1.5, top-p 0.95; nucleus
// sampling is its reference [18]).
//
// bf16 rows, one pass over HBM.  A bf16 logit takes one of 65536 values and
// every token with the same value has the same probability, so the exact count
// of tokens per value determines the maximum, sum_v exp(l_v/T) and the top-p
// cut (the first value, from the top, at which the cumulative mass reaches
// top_p).  The counts go into an LDS histogram with one bin per bf16 value of
// magnitude in [2^-24, 2^24) (48 binades x 128 mantissas per sign = 12288
// bins), two 16-bit counters per 32-bit word (24 KiB).  Integer counts are
// exact and order-independent, so the result is deterministic.  A 16-bit
// counter can wrap only if one value holds >= 65536 tokens; then the counts no
// longer sum to V, which is checked.  The masses count * exp(v/T - m/T) are
// formed once per non-empty bin in double: one wave takes 64 consecutive bins
// (one per lane), so the exp work is spread evenly; the row totals are scanned
// to find the 64-bin row holding the top_p crossing, and one wave rescans that
// row.  Rows holding a value outside the histogram range (zero, |l| < 2^-24,
// |l| >= 2^24, NaN, Inf), or a wrapped counter, take the generic path instead.
//
// Generic path (fp32 rows, or those bf16 rows): max and argmax, then sum
// exp(l/T - m/T) in double, then the cut by bisection over the monotone 32-bit
// key of the values (at most 32 passes over the row, which stays in cache).
#pragma once

#include <math.h>

#include "sv_device.hpp"

namespace sv {

constexpr uint32_t kExpLo = 103u << 7;     // |v| >= 2^-24: biased exponent 103
constexpr int kSide = 6144;                // 48 exponents x 128 mantissas
constexpr int kNBins = 2 * kSide + 2;      // [0] negative special, [1..6144] negative values,
                                           // [6145..12288] positive values, [12289] positive special
constexpr int kHistWords = kNBins / 2;     // two 16-bit counters per word
constexpr int kMassRows = 2 * kSide / 64;  // 64-bin rows of the in-range bins

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
  float* row_cut;        // NULL when only statistics are wanted
  double* row_kept_lse;  // NULL when only statistics are wanted
  uint32_t* status;
  // Optional copies for the fused draw: row j of request r also goes to
  // slot[r * (slot_b + 1) + j] (j <= slot_b), with the logit at draft token
  // gx[r * slot_b + j] when the row has one (target rows, row_stride 0: j <
  // L_r; draft rows, row_stride b: every row).  slot_at: the slot of the
  // block's row (set per block; -1: none).
  SlotRec* slot;
  const int32_t* gx;
  int slot_b;
  int slot_at = -1;
};

template <int NT>
struct RowShared {
  uint64_t red_u64[NT / kWave];
  double red_f64[NT / kWave];
  int red_i32[NT / kWave];
  double rowtot[kMassRows];
  double etab[kExpTab];  // the exponential's table (exp_table_init at the kernel's start)
  int req;
  int cut_d;
  double F;
};

__device__ inline void write_row(const RowArgs& a, int p, float mx, int am, double lse, float cut, double kept) {
  a.row_max[p] = mx;
  a.row_argmax[p] = am;
  a.row_lse[p] = lse;
  if (a.row_cut) a.row_cut[p] = cut;
  if (a.row_kept_lse) a.row_kept_lse[p] = kept;
  if (a.slot != nullptr && a.slot_at >= 0) {
    SlotRec& sr = a.slot[a.slot_at];
    sr.kept = kept;
    sr.cut = cut;
    sr.argmax = am;
  }
}

__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin) {
  atomicAdd(&hist[bin >> 1], 1u << ((bin & 1u) << 4));
}

__device__ __forceinline__ uint32_t hist_get(const uint32_t* hist, int bin) {
  return (hist[bin >> 1] >> ((bin & 1) << 4)) & 0xFFFFu;
}

// ------------------------------------------------------------------ generic path
template <int DT, int NT>
__device__ void row_generic(const RowArgs& a, const void* rowp, int p, float T, float tp, bool topp_on,
                            RowShared<NT>& sh) {
  const int tid = threadIdx.x;
  const int V = a.V;
  float best = -INFINITY;
  int bidx = -1;
  bool nonfinite = false;
  for (int v = tid; v < V; v += NT) {
    const float f = load_val<DT>(rowp, v);
    nonfinite |= !isfinite(f);
    if (f > best) {
      best = f;
      bidx = v;
    }
  }
  if (nonfinite) raise_status(a.status, SV_ST_NONFINITE);
  uint64_t packed = bidx >= 0 ? (static_cast<uint64_t>(mono_key(best)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bidx)) : 0;
  packed = block_max_u64<NT>(packed, sh.red_u64);
  const float m = packed ? key_value(static_cast<uint32_t>(packed >> 32)) : -INFINITY;
  const int am = packed ? static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(packed)) : 0;
  if (T == 0.0f) {
    if (tid == 0) write_row(a, p, m, am, 0.0, m, 0.0);
    return;
  }
  const double Td = static_cast<double>(T);
  const double M = static_cast<double>(m) / Td;
  double part = 0.0;
  for (int v = tid; v < V; v += NT) part += exp(static_cast<double>(load_val<DT>(rowp, v)) / Td - M);
  const double Z = block_sum_f64<NT>(part, sh.red_f64);
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
    for (int v = tid; v < V; v += NT) {
      const float f = load_val<DT>(rowp, v);
      if (mono_key(f) >= mid) s += exp(static_cast<double>(f) / Td - M);
    }
    const double F = block_sum_f64<NT>(s, sh.red_f64);
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
  hist_add(hist, bb.x & 0xFFFFu);
  hist_add(hist, bb.x >> 16);
  hist_add(hist, bb.y & 0xFFFFu);
  hist_add(hist, bb.y >> 16);
  hist_add(hist, bb.z & 0xFFFFu);
  hist_add(hist, bb.z >> 16);
  hist_add(hist, bb.w & 0xFFFFu);
  hist_add(hist, bb.w >> 16);
  const u16x2 m2 = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, bb.x), __builtin_bit_cast(u16x2, bb.y)),
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, bb.z), __builtin_bit_cast(u16x2, bb.w)));
  vmax = m2.x > m2.y ? m2.x : m2.y;
}

// Mass of in-range bin number d in descending order (d = 0 is bin 12288).
__device__ __forceinline__ double bin_mass(const uint32_t* hist, int d, double Td, double M, const double* tab) {
  const int bin = 2 * kSide - d;
  const uint32_t c = hist_get(hist, bin);
  double m = 0.0;
  if (c) m = static_cast<double>(c) * exp_tab(static_cast<double>(bin_value(bin)) / Td - M, tab);
  return m;
}

template <int DT, int NT, int BATCH, bool kBatchCheck = true>
__device__ __forceinline__ void row_stats_at(const RowArgs& a, const void* rowp, int p, float T, float tp, bool topp_on,
                             uint32_t* hist, RowShared<NT>& sh);

// Where row p (work item p of the request found from row_off) lies and how it
// is filtered; ok = false if the offsets are malformed (status raised).
struct RowLoc {
  bool ok, topp_on;
  const void* rowp;
  float T, tp;
  int r, j;  // request, and the row's index within it
};

template <int DT, int NT>
__device__ __forceinline__ RowLoc row_locate(const RowArgs& a, int p, RowShared<NT>& sh) {
  RowLoc l{false, false, nullptr, 0.0f, 1.0f, -1, -1};
  const int tid = threadIdx.x;
  const int r = find_request<NT>(a.row_off, a.R, p, &sh.req);
  if (r < 0) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return l;
  }
  const int j = p - a.row_off[r];
  l.r = r;
  l.j = j;
  if (a.row_stride > 0 && j >= a.row_stride) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_OFFSETS);
    return l;
  }
  const int64_t row = a.row_stride > 0 ? static_cast<int64_t>(r) * a.row_stride + j : static_cast<int64_t>(p);
  const size_t esz = DT == SV_BF16 ? 2 : 4;
  l.rowp = static_cast<const char*>(a.logits) + static_cast<size_t>(row) * static_cast<size_t>(a.ld) * esz;
  l.T = a.T[r];
  l.tp = a.top_p ? a.top_p[r] : 1.0f;
  if (tid == 0 && !(l.T >= 0.0f)) raise_status(a.status, SV_ST_BAD_TEMPERATURE);
  l.topp_on = a.row_cut != nullptr && a.top_p != nullptr && !(l.tp >= 1.0f);
  if (l.topp_on && !(l.tp > 0.0f)) {
    if (tid == 0) raise_status(a.status, SV_ST_BAD_TOP_P);
    l.tp = 1e-30f;  // keeps the top value only
  }
  l.ok = true;
  return l;
}

// a with the slot of the located row (uniform, so kept in scalar registers)
__device__ __forceinline__ RowArgs with_slot(const RowArgs& a, const RowLoc& l) {
  RowArgs s = a;
  s.slot_at = a.slot != nullptr && l.j >= 0 && l.j <= a.slot_b
                  ? __builtin_amdgcn_readfirstlane(l.r * (a.slot_b + 1) + l.j)
                  : -1;
  return s;
}

// The located row's logit at its draft token into its slot, if it has one
// (one thread; a token outside the vocabulary reads element 0 here, and the
// draw reports it).
template <int DT>
__device__ __forceinline__ void slot_gather(const RowArgs& s, const RowLoc& l) {
  if (s.slot_at < 0 || l.j >= s.slot_b) return;
  const int n = s.row_off[l.r + 1] - s.row_off[l.r] - (s.row_stride > 0 ? 0 : 1);  // rows with a draft token
  if (l.j >= n) return;
  const int x = s.gx[static_cast<size_t>(l.r) * s.slot_b + l.j];
  s.slot[s.slot_at].lx = load_val<DT>(l.rowp, x >= 0 && x < s.V ? x : 0);
}

// Statistics of row p (work item p of the request found from row_off), by one
// block of NT threads.  `hist` holds kHistWords words of LDS (bf16 rows only).
template <int DT, int NT, int BATCH, bool kBatchCheck = true>
__device__ void row_block(const RowArgs& a, int p, uint32_t* hist, RowShared<NT>& sh) {
  const RowLoc l = row_locate<DT, NT>(a, p, sh);
  if (!l.ok) return;
  const RowArgs s = with_slot(a, l);
  row_stats_at<DT, NT, BATCH, kBatchCheck>(s, l.rowp, p, l.T, l.tp, l.topp_on, hist, sh);
  // by the last wave (the first to finish its part of the statistics)
  if (threadIdx.x == NT - 1) slot_gather<DT>(s, l);
}

// ------------------------------------------------------------------ bf16 streaming path (no cut)
// Maximum, argmax (lowest index) and sum_v exp(l_v / T) of a bf16 row, or of
// the vectors [v0, v1) of it, in one pass, when no top-p cut is wanted (the
// histogram's LDS atomics would only cost time).  Each thread keeps a running
// maximum m and a sum of exp((l - m) / T), rescaled in double when m grows;
// a full batch of BATCH vectors is checked once (its maximum first, then all
// its exponentials in the frame that maximum sets: one branch per batch, so
// the exponentials of the batch issue back to back);
// the 8 values of a 16-byte vector are exponentiated in fp32 (the hardware
// exp2 of (l - m) * log2(e) / T; a term below 2^-126 of the running maximum
// may flush to 0, far below the sum's rounding) and summed in fp32, the
// vector sums in double; the block combines the threads' sums in double
// (fp32 accumulation, as the row statistics are specified).  Output: the
// block maximum M, the packed argmax key (order key of the value above the
// complemented index; 0 if the range is empty) and S = sum exp2((l - M) * c2)
// with c2 = log2(e) / T, so that lse = M / T + log(S).  T = 0: M and the key
// only (S = 0).  NaN and +-Inf raise SV_ST_NONFINITE.  `tail`: the elements past
// the last full vector belong to this range.
struct StreamPart {
  float M;
  uint64_t key;
  double S;
};

__device__ __forceinline__ float soft_c2(float T) { return T > 0.0f ? 1.4426950408889634f / T : 0.0f; }

// Maximum of three values as the hardware's v_max3_f32 forms it, without the
// quieting of signalling NaNs that fmaxf adds before each maximum: a NaN
// value still reaches the sums, which report it.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int NT, int BATCH, bool kBatchCheck = true>
__device__ __forceinline__ StreamPart stream_part_bf16(const uint16_t* rp, int V, int v0, int v1, bool tail, float T,
                                                       uint32_t* status, RowShared<NT>& sh) {
  const int tid = threadIdx.x;
  const uint4* vp = reinterpret_cast<const uint4*>(rp);
  const int nvec = V >> 3;
  const bool sums = T > 0.0f;
  const float c2 = soft_c2(T);  // log2(e) / T
  // The thread's terms are exp2(fma(l, c2, -mc)) with mc = fl(m * c2): the
  // frame mc changes (exactly, in double) when m grows; the block frame is
  // M * c2 in double.
  float m = -INFINITY, mc = -INFINITY, mn = INFINITY;
  u16x2 hw = {0, 0};  // largest raw halves of the full batches: -inf (0xFF80) and negative NaNs at or above it
  // T = 0 forms no sums, so NaN cannot show there: the largest magnitude half
  // (sign bit cleared) of every vector is kept instead; >= 0x7F80 is +-inf or NaN
  u16x2 hz = {0, 0};
  const uint32_t kMag = 0x7FFF7FFFu;
  auto mags = [&](const uint4& d) {
    hz = __builtin_elementwise_max(
        hz, __builtin_elementwise_max(
                __builtin_elementwise_max(__builtin_bit_cast(u16x2, d.x & kMag), __builtin_bit_cast(u16x2, d.y & kMag)),
                __builtin_elementwise_max(__builtin_bit_cast(u16x2, d.z & kMag), __builtin_bit_cast(u16x2, d.w & kMag))));
  };
  double s = 0.0;
  int bvi = -1;
  uint4 bv = {0, 0, 0, 0};
  auto take = [&](const uint4& d, int vi) {
    float v[8];
    v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x); v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
    v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z); v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
    const float vm = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])), fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
    mn = fminf(fminf(mn, fminf(v[0], v[1])), fminf(fminf(v[2], v[3]), fminf(v[4], v[5])));
    mn = fminf(mn, fminf(v[6], v[7]));
    if (vm > m) {  // rare after the first vectors: the frame change runs in double
      const float mcn = vm * c2;
      if (sums) s *= exp2(static_cast<double>(mc) - static_cast<double>(mcn));  // 0 while m = -inf
      m = vm;
      mc = mcn;
      bvi = vi;
      bv = d;
    }
    if (sums) {
      float acc = __builtin_amdgcn_exp2f(fmaf(v[0], c2, -mc));
#pragma unroll
      for (int q = 1; q < 8; ++q) acc += __builtin_amdgcn_exp2f(fmaf(v[q], c2, -mc));
      s += static_cast<double>(acc);
    } else {
      mags(d);
    }
  };
  int v = v0 + tid;
  // unconditional loads, indices clamped to the range's last vector (re-read,
  // unused): no branch makes the compiler wait for the batch in flight
  const int last = v1 - 1;
  uint4 cur[BATCH];
  if (v1 > v0) {
#pragma unroll
    for (int k = 0; k < BATCH; ++k) cur[k] = load16_stream(vp + min(v + k * NT, last));
  }
  while (v < v1) {
    const int vn = v + BATCH * NT;
    uint4 nxt[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) nxt[k] = load16_stream(vp + min(vn + k * NT, last));
    if (!kBatchCheck && v + (BATCH - 1) * NT < v1) {  // a full batch, one check per vector (fewer registers)
#pragma unroll
      for (int k = 0; k < BATCH; ++k) take(cur[k], v + k * NT);
    } else if (v + (BATCH - 1) * NT < v1) {  // a full batch: one frame check for its vectors
      float vmx[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        const uint4& d = cur[k];
        float w[8];
        w[0] = bf16_lo(d.x); w[1] = bf16_hi(d.x); w[2] = bf16_lo(d.y); w[3] = bf16_hi(d.y);
        w[4] = bf16_lo(d.z); w[5] = bf16_hi(d.z); w[6] = bf16_lo(d.w); w[7] = bf16_hi(d.w);
        vmx[k] = max3_raw(max3_raw(w[0], w[1], w[2]), max3_raw(w[3], w[4], w[5]), max3_raw(w[6], w[7], w[7]));
        hw = __builtin_elementwise_max(
            hw, __builtin_elementwise_max(
                    __builtin_elementwise_max(__builtin_bit_cast(u16x2, d.x), __builtin_bit_cast(u16x2, d.y)),
                    __builtin_elementwise_max(__builtin_bit_cast(u16x2, d.z), __builtin_bit_cast(u16x2, d.w))));
      }
      float bm = vmx[0];
#pragma unroll
      for (int k = 1; k < BATCH; k += 2) bm = max3_raw(bm, vmx[k], vmx[k + 1 < BATCH ? k + 1 : k]);
      if (bm > m) {
        bool found = false;
#pragma unroll
        for (int k = 0; k < BATCH; ++k)
          if (!found && vmx[k] == bm) {
            found = true;
            bvi = v + k * NT;
            bv = cur[k];
          }
        const float mcn = bm * c2;
        if (sums) s *= exp2(static_cast<double>(mc) - static_cast<double>(mcn));
        m = bm;
        mc = mcn;
      }
      if (sums) {
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
          const uint4& d = cur[k];
          float w[8];
          w[0] = bf16_lo(d.x); w[1] = bf16_hi(d.x); w[2] = bf16_lo(d.y); w[3] = bf16_hi(d.y);
          w[4] = bf16_lo(d.z); w[5] = bf16_hi(d.z); w[6] = bf16_lo(d.w); w[7] = bf16_hi(d.w);
          float acc = __builtin_amdgcn_exp2f(fmaf(w[0], c2, -mc));
#pragma unroll
          for (int q = 1; q < 8; ++q) acc += __builtin_amdgcn_exp2f(fmaf(w[q], c2, -mc));
          s += static_cast<double>(acc);
        }
      } else {
#pragma unroll
        for (int k = 0; k < BATCH; ++k) mags(cur[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < BATCH; ++k)
        if (v + k * NT < v1) take(cur[k], v + k * NT);
    }
#pragma unroll
    for (int k = 0; k < BATCH; ++k) cur[k] = nxt[k];
    v = vn;
  }
  int bidx = -1;
  float best = m;
  if (bvi >= 0) {
    const float e[8] = {bf16_lo(bv.x), bf16_hi(bv.x), bf16_lo(bv.y), bf16_hi(bv.y),
                        bf16_lo(bv.z), bf16_hi(bv.z), bf16_lo(bv.w), bf16_hi(bv.w)};
    int k = 7;
#pragma unroll
    for (int q = 7; q >= 0; --q)
      if (e[q] == best) k = q;
    bidx = bvi * 8 + k;
  }
  if (tail) {
    for (int e = (nvec << 3) + tid; e < V; e += NT) {  // elements past the last full vector
      const float f = __uint_as_float(static_cast<uint32_t>(rp[e]) << 16);
      if (!(f == f)) hz.x = 0x7FFFu;  // NaN (a tail element; T = 0 forms no sum to show it)
      mn = fminf(mn, f);
      if (f > m) {
        const float mcn = f * c2;
        if (sums) s *= exp2(static_cast<double>(mc) - static_cast<double>(mcn));
        m = f;
        mc = mcn;
      }
      if (f > best || bidx < 0) {
        best = f;
        bidx = e;
      }
      if (sums) s += static_cast<double>(__builtin_amdgcn_exp2f(fmaf(f, c2, -mc)));
    }
  }
  if (mn == -INFINITY || hw.x >= 0xFF80u || hw.y >= 0xFF80u || hz.x >= 0x7F80u || hz.y >= 0x7F80u)
    raise_status(status, SV_ST_NONFINITE);
  uint64_t packed =
      bidx >= 0 ? (static_cast<uint64_t>(mono_key(best)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bidx)) : 0;
  StreamPart out;
  out.key = block_max_u64<NT>(packed, sh.red_u64);
  out.M = out.key ? key_value(static_cast<uint32_t>(out.key >> 32)) : -INFINITY;
  out.S = 0.0;
  if (sums) {  // this thread's sum moved to the block frame M * c2, in double
    const double part =
        m > -INFINITY ? s * exp2(static_cast<double>(mc) - static_cast<double>(out.M) * static_cast<double>(c2)) : 0.0;
    out.S = block_sum_f64<NT>(part, sh.red_f64);
  }
  if (tid == 0 && !(out.M < INFINITY && out.S < INFINITY)) raise_status(status, SV_ST_NONFINITE);
  return out;
}

// Statistics of the row at `rowp` at temperature T (top-p cut when topp_on),
// written to output slot p of a's arrays, by one block of NT threads.
template <int DT, int NT, int BATCH, bool kBatchCheck>
__device__ __forceinline__ void row_stats_at(const RowArgs& a, const void* rowp, int p, float T, float tp, bool topp_on,
                             uint32_t* hist, RowShared<NT>& sh) {
  const int tid = threadIdx.x;
  if constexpr (DT == SV_BF16) {
    if (!topp_on) {  // no cut wanted: one streaming pass
      const StreamPart sp =
          stream_part_bf16<NT, BATCH, kBatchCheck>(static_cast<const uint16_t*>(rowp), a.V, 0, a.V >> 3, true, T,
                                                   a.status, sh);
      if (tid == 0) {
        const int am = static_cast<int>(argmax_token(sp.key));
        if (T == 0.0f)
          write_row(a, p, sp.M, am, 0.0, sp.M, 0.0);
        else {
          const double lse = static_cast<double>(sp.M) / static_cast<double>(T) + log(sp.S);
          write_row(a, p, sp.M, am, lse, -INFINITY, lse);
        }
      }
      return;
    }
    for (int k = tid; k < kHistWords; k += NT) hist[k] = 0u;
    __syncthreads();
    const uint16_t* rp = static_cast<const uint16_t*>(rowp);
    const uint4* vp = reinterpret_cast<const uint4*>(rp);
    const int nvec = a.V >> 3;
    uint32_t best = 0;
    int bvec = -1;
    uint4 bbins = {0, 0, 0, 0};
    int v = tid;
    const int last = nvec - 1;  // unconditional, clamped loads (see stream_row_bf16)
    uint4 cur[BATCH];
    if (nvec > 0) {
#pragma unroll
      for (int k = 0; k < BATCH; ++k) cur[k] = load16_stream(vp + min(v + k * NT, last));
    }
    while (v < nvec) {
      const int vn = v + BATCH * NT;
      uint4 nxt[BATCH];
#pragma unroll
      for (int k = 0; k < BATCH; ++k) nxt[k] = load16_stream(vp + min(vn + k * NT, last));
#pragma unroll
      for (int k = 0; k < BATCH; ++k) {
        if (v + k * NT < nvec) {
          uint4 bb;
          uint32_t vm;
          count_vec(hist, cur[k], bb, vm);
          if (vm > best) {
            best = vm;
            bvec = v + k * NT;
            bbins = bb;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < BATCH; ++k) cur[k] = nxt[k];
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
    for (int e = (nvec << 3) + tid; e < a.V; e += NT) {  // elements past the last full vector
      const uint32_t bn = bin_of(rp[e]);
      hist_add(hist, bn);
      if (bn > best || bidx < 0) {
        best = bn;
        bidx = e;
      }
    }
    uint64_t packed = bidx >= 0 ? (static_cast<uint64_t>(best) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(bidx)) : 0;
    packed = block_max_u64<NT>(packed, sh.red_u64);  // its barriers also complete the histogram
    int csum = 0;
    for (int k = tid; k < kHistWords; k += NT) csum += static_cast<int>((hist[k] & 0xFFFFu) + (hist[k] >> 16));
    int ctot;
    (void)block_excl_scan_i32<NT>(csum, sh.red_i32, &ctot);
    const uint32_t special = hist_get(hist, 0) + hist_get(hist, kNBins - 1);
    if (special == 0u && ctot == a.V) {
      const int mbin = static_cast<int>(packed >> 32);
      const int am = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(packed));
      const float m = bin_value(mbin);
      if (T == 0.0f) {
        if (tid == 0) write_row(a, p, m, am, 0.0, m, 0.0);
        return;
      }
      const double Td = static_cast<double>(T);
      const double M = static_cast<double>(m) / Td;
      // masses: wave w takes 64-bin rows w, w + NW, ...; one bin per lane
      constexpr int NW = NT / kWave;
      const int lane = tid & (kWave - 1), wv = tid / kWave;
      for (int rr = wv; rr < kMassRows; rr += NW) {
        // a 64-bin row with no token (most rows outside the values' binades) skips the exp
        const double tot = __ballot(hist_get(hist, 2 * kSide - (rr * kWave + lane)) != 0u)
                               ? wave_sum_f64(bin_mass(hist, rr * kWave + lane, Td, M, sh.etab))
                               : 0.0;
        if (lane == 0) sh.rowtot[rr] = tot;
      }
      __syncthreads();
      if (wv != 0) return;
      // wave 0: scan the row totals (3 per lane, in descending order), then the crossing row
      constexpr int RPL = kMassRows / kWave;
      static_assert(RPL * kWave == kMassRows, "row totals must split evenly over a wave");
      double rt[RPL];
      double loc = 0.0;
#pragma unroll
      for (int k = 0; k < RPL; ++k) {
        rt[k] = sh.rowtot[lane * RPL + k];
        loc += rt[k];
      }
      const double inc = wave_incl_scan_f64(loc);
      const double Z = bcast_f64(inc, kWave - 1);
      const double lse = M + log(Z);
      if (!topp_on) {
        if (lane == 0) write_row(a, p, m, am, lse, -INFINITY, lse);
        return;
      }
      const double target = static_cast<double>(tp) * Z;
      const uint64_t over = __ballot(inc >= target);
      if (!over) {  // rounding kept the cumulative mass below target: keep every token
        int low = -1;
        for (int d = lane; d < 2 * kSide; d += kWave)
          if (hist_get(hist, 2 * kSide - d)) low = d;
        low = wave_max_i32(low);
        if (lane == 0) write_row(a, p, m, am, lse, bin_value(2 * kSide - low), lse);
        return;
      }
      const int cl = __ffsll(static_cast<long long>(over)) - 1;
      // within lane cl's rows, the first whose running total reaches target
      // (its last row if rounding keeps them all below)
      int crow = 0;
      double cbase = 0.0;
      if (lane == cl) {
        double run = inc - loc;
        for (int k = 0; k < RPL; ++k) {
          if (run + rt[k] >= target || k == RPL - 1) {
            crow = cl * RPL + k;
            cbase = run;
            break;
          }
          run += rt[k];
        }
      }
      crow = bcast_i32(crow, cl);
      cbase = bcast_f64(cbase, cl);
      const double mass = bin_mass(hist, crow * kWave + lane, Td, M, sh.etab);
      const double inc2 = cbase + wave_incl_scan_f64(mass);
      const uint64_t hit = __ballot(inc2 >= target);
      int cut_d;
      double F;
      if (hit) {
        const int hl = __ffsll(static_cast<long long>(hit)) - 1;
        cut_d = crow * kWave + hl;
        F = bcast_f64(inc2, hl);
      } else {  // rounding: the last non-empty bin of the row
        const uint64_t ne = __ballot(mass > 0.0 || hist_get(hist, 2 * kSide - (crow * kWave + lane)) != 0u);
        const int hl = ne ? 63 - __clzll(static_cast<long long>(ne)) : kWave - 1;
        cut_d = crow * kWave + hl;
        F = bcast_f64(inc2, kWave - 1);
      }
      if (lane == 0) write_row(a, p, m, am, lse, bin_value(2 * kSide - cut_d), M + log(F));
      return;
    }
    // a value outside the histogram range, or a wrapped counter: exact generic path
    row_generic<SV_BF16, NT>(a, rowp, p, T, tp, topp_on, sh);
  } else {
    row_generic<SV_F32, NT>(a, rowp, p, T, tp, topp_on, sh);
  }
}

}  // namespace sv
