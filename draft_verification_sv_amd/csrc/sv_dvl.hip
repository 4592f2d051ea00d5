// sv_dvl.hip -- dynamic verify-length (DVL) allocation and packing.
//
// "DScale: Scaling Block-Diffusion Speculative Decoding with Adaptive
// Verification", abstract: a budget of verification slots -- half of what the
// engine could verify at full length -- goes to the draft prefixes with the
// best scores, and the per-request lengths reach the verification kernels
// through buffers at fixed addresses.  A prefix is scored by the probability
// that it survives verification (wispaper Q&A on block-diffusion decode
// failures, section "Why does throughput collapse under high concurrency?",
// on DSpark): s_{r,i} = a_{r,1} * ... * a_{r,i}, one float rounding per
// product.  The allocation keeps the B highest scores in the order (s desc, r
// asc, i asc); with a <= 1 the scores fall along each request, so the choice is
// prefix-closed and maximises the summed survival (expected accepted length).
//
// Per-request block length (wispaper Q&A on block-diffusion decode failures,
// section "Why is a fixed block size a failure mode in production?": BlockPilot
// finds the best block size varies per request): with block_len, request r
// drafted only its first b_r positions; the others are not candidates and get s = 0.  The
// selection key of a candidate is its score key + 1 and that of any other
// position 0, and the budget is capped at sum_r b_r, so the threshold is >= 1
// and never admits a non-candidate.  Without block_len every key is shifted
// alike and the result is unchanged.
//
// One block of kDvlNT = 512 threads:
//   1. per request, the running products (written to s);
//   2. radix select, 10 bits per pass from the top (three passes: selection
//      keys are below 2^30), of the B-th largest score (score bits with -0
//      read as +0: non-negative floats order like their bit patterns), with
//      LDS count histograms; the digit holding the rank is
//      found by a block scan over the 1024 digit counts; then a position is
//      taken if above the threshold or a tie of rank below the remainder in
//      (r, i) order (an exclusive scan of tie counts);
//   3. L_r counted with integer atomics;
//   4. exclusive scans of L and L + 1 into pos_off and tgt_off.
#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

// order key of a non-negative score: its bits, with -0 read as +0
__device__ __forceinline__ uint32_t score_key(float v) {
  const uint32_t k = __float_as_uint(v);
  return k == 0x80000000u ? 0u : k;
}

// selection key of a drafted position: score key + 1, with keys above that
// of 1.0 (only from estimates outside [0, 1], which raise a status bit) held
// at it, so that every key is below 2^30
__device__ __forceinline__ uint32_t select_key(float v) { return min(score_key(v), 0x3F800000u) + 1u; }

constexpr int kDigitBits = 10;            // three radix passes cover the 30 key bits
constexpr int kBins = 1 << kDigitBits;

constexpr int kDvlNT = 512;  // 8 waves: 5.5 us a call at R = 32, b = 16 against 6.0 (256), 7.2 (128), 6.4 (1024)
constexpr int kDvlLds = 8192;  // scores kept in LDS up to this many positions

// b_r of request r: block_len[r] clamped to [0, b] (b without block_len)
__device__ __forceinline__ int block_of(const int32_t* block_len, int r, int b) {
  return block_len ? min(max(block_len[r], 0), b) : b;
}

template <bool kInLds>
__global__ __launch_bounds__(kDvlNT) void k_dvl(const float* __restrict__ a, int R, int b,
                                               const int32_t* __restrict__ block_len,
                                               const int32_t* __restrict__ budget, float* __restrict__ s,
                                               int32_t* __restrict__ L, int32_t* __restrict__ pos_off,
                                               int32_t* __restrict__ tgt_off, uint32_t* status) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t skey[kInLds ? kDvlLds : 1];
  __shared__ int scr[kDvlNT / kWave];
  __shared__ int lcount[kInLds ? kDvlLds : 1];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_remaining;
  const int tid = threadIdx.x;
  const int n = R * b;
  int B = *budget;
  if (B < 0) {
    if (tid == 0) raise_status(status, SV_ST_BAD_BUDGET);
    B = 0;
  }
  // candidates: sum_r b_r
  int n_cand = n;
  if (block_len) {
    const int pr0 = (R + kDvlNT - 1) / kDvlNT;
    int c = 0;
    bool bad_bl = false;
    for (int r = tid * pr0; r < min(R, (tid + 1) * pr0); ++r) {
      const int v = block_len[r];
      bad_bl |= v < 0 || v > b;
      c += min(max(v, 0), b);
    }
    if (bad_bl) raise_status(status, SV_ST_BAD_BLOCK);
    (void)block_excl_scan_i32<kDvlNT>(c, scr, &n_cand);
  }
  // 1. survival scores.  The estimates are read in one coalesced pass (into
  // LDS when they fit) before any score is written, so no load waits behind a
  // store.
  bool bad = false;
  if constexpr (kInLds) {
    for (int e = tid; e < n; e += kDvlNT) skey[e] = __float_as_uint(a[e]);
    for (int r = tid; r < R; r += kDvlNT) lcount[r] = 0;
    __syncthreads();
    // per request: the running products in place, the estimates checked;
    // positions past b_r marked (no score has these bits)
    for (int r = tid; r < R; r += kDvlNT) {
      const int br = block_of(block_len, r, b);
      float run = 1.0f;
      for (int i = 0; i < b; ++i) {
        const float av = __uint_as_float(skey[r * b + i]);
        bad |= i < br && !(av >= 0.0f && av <= 1.0f);
        run = run * av;
        skey[r * b + i] = i < br ? __float_as_uint(run) : 0xFFFFFFFFu;
      }
    }
    __syncthreads();
    for (int e = tid; e < n; e += kDvlNT) {
      const bool cand = skey[e] != 0xFFFFFFFFu;
      const float sv = cand ? __uint_as_float(skey[e]) : 0.0f;
      s[e] = sv;
      skey[e] = cand ? select_key(sv) : 0u;
    }
  } else {
    for (int r = tid; r < R; r += kDvlNT) L[r] = 0;
    for (int r = tid; r < R; r += kDvlNT) {
      const int br = block_of(block_len, r, b);
      float run = 1.0f;
      for (int i = 0; i < b; ++i) {
        const float av = a[r * b + i];
        bad |= i < br && !(av >= 0.0f && av <= 1.0f);
        run = run * av;
        s[r * b + i] = i < br ? run : 0.0f;
      }
    }
  }
  if (bad) raise_status(status, SV_ST_BAD_SCORE);
  __syncthreads();  // scores are re-read below by other threads of this block
  const bool all = B >= n_cand, none = B == 0;

  {
    // selection key: score key + 1 for a candidate, 0 past b_r
    auto key = [&](int e) -> uint32_t {
      if constexpr (kInLds) return skey[e];
      else return (e % b) < block_of(block_len, e / b, b) ? select_key(s[e]) : 0u;
    };
    // 2. threshold: the B-th largest score (rank from the top, ties counted)
    uint32_t thr = 0;
    int remaining = 0;  // how many ties at thr are taken
    if (!all && !none) {
      uint32_t prefix = 0, mask = 0;
      remaining = B;
      constexpr int kPerThread = kBins / kDvlNT;
      static_assert(kPerThread * kDvlNT == kBins, "digits must split evenly over the block");
      for (int shift = 2 * kDigitBits; shift >= 0; shift -= kDigitBits) {
        for (int k = tid; k < kBins; k += kDvlNT) hist[k] = 0u;
        __syncthreads();
        for (int e = tid; e < n; e += kDvlNT) {
          const uint32_t kk = key(e);
          if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & (kBins - 1)], 1u);
        }
        __syncthreads();
        // digits from the top: thread t holds digits kBins-1 - (t*kPerThread + j);
        // the crossing digit is the one whose exclusive count from the top is
        // < remaining <= inclusive
        int h[kPerThread], hs = 0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
          h[j] = static_cast<int>(hist[kBins - 1 - (tid * kPerThread + j)]);
          hs += h[j];
        }
        int tot;
        const int excl = block_excl_scan_i32<kDvlNT>(hs, scr, &tot);
        if (excl < remaining && remaining <= excl + hs) {
          int run = excl;
#pragma unroll
          for (int j = 0; j < kPerThread; ++j) {
            if (run < remaining && remaining <= run + h[j]) {
              sh_prefix = prefix | (static_cast<uint32_t>(kBins - 1 - (tid * kPerThread + j)) << shift);
              sh_remaining = remaining - run;
            }
            run += h[j];
          }
        }
        __syncthreads();
        prefix = sh_prefix;
        remaining = sh_remaining;
        mask |= static_cast<uint32_t>(kBins - 1) << shift;
      }
      thr = prefix;
    }
    // 3. element-parallel choice: above the threshold, or a tie whose rank in
    // (r, i) order is below `remaining`; lengths counted with atomics.
    // Thread t owns the consecutive elements [t*pe, (t+1)*pe).
    const int pe = (n + kDvlNT - 1) / kDvlNT;
    const int e0 = tid * pe, e1 = min(n, e0 + pe);
    int eq_local = 0;
    if (!all && !none)
      for (int e = e0; e < e1; ++e) eq_local += key(e) == thr ? 1 : 0;
    int eq_total;
    int tie_rank = block_excl_scan_i32<kDvlNT>(eq_local, scr, &eq_total);
    for (int e = e0; e < e1; ++e) {
      bool take;
      if (all) {
        take = key(e) != 0u;
      } else if (none) {
        take = false;
      } else {
        const uint32_t kk = key(e);
        take = kk > thr || (kk == thr && tie_rank < remaining);
        tie_rank += kk == thr ? 1 : 0;
      }
      if (take) {
        if constexpr (kInLds)
          atomicAdd(&lcount[e / b], 1);
        else
          atomicAdd(&L[e / b], 1);
      }
    }
  }
  __syncthreads();
  // 4. lengths and offsets: thread t owns the consecutive requests [t*pr, (t+1)*pr)
  const int pr = (R + kDvlNT - 1) / kDvlNT;
  const int r0 = tid * pr, r1 = min(R, r0 + pr);
  int l_local = 0;
  auto length = [&](int r) -> int {
    if constexpr (kInLds) return lcount[r];
    else return __hip_atomic_load(&L[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  for (int r = r0; r < r1; ++r) l_local += length(r);
  int l_total;
  int off = block_excl_scan_i32<kDvlNT>(l_local, scr, &l_total);
  for (int r = r0; r < r1; ++r) {
    const int Lr = length(r);
    if constexpr (kInLds) L[r] = Lr;
    pos_off[r] = off;
    tgt_off[r] = off + r;
    off += Lr;
  }
  if (tid == 0) {
    pos_off[R] = l_total;
    tgt_off[R] = l_total + R;
  }
}

}  // namespace sv

using namespace sv;

extern "C" int32_t dvl_alloc_pack(const float* a, int32_t R, int32_t b, const int32_t* block_len,
                                  const int32_t* budget, float* s, int32_t* L, int32_t* pos_off, int32_t* tgt_off,
                                  void* ws, size_t ws_bytes, void* stream) {
  if (!a || !budget || !s || !L || !pos_off || !tgt_off || !ws) return SV_ERR_ARG;
  if (R < 1 || b < 1 || b > 64 || static_cast<long long>(R) * b > (1LL << 24)) return SV_ERR_ARG;
  if (ws_bytes < 256) return SV_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (R * b <= kDvlLds)
    hipLaunchKernelGGL(k_dvl<true>, dim3(1), dim3(kDvlNT), 0, st, a, R, b, block_len, budget, s, L, pos_off,
                       tgt_off, status_word(ws));
  else
    hipLaunchKernelGGL(k_dvl<false>, dim3(1), dim3(kDvlNT), 0, st, a, R, b, block_len, budget, s, L, pos_off,
                       tgt_off, status_word(ws));
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
