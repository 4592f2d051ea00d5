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

// ------------------------------------------------------------------ short-block path
// When b divides 64, R <= 64 and R * b <= NT (R = 32, b = 16 at the largest
// configuration), each request's positions are consecutive lanes of one
// wave, and the whole call is a few wave-level steps with seven block
// barriers (the general kernel above takes about twenty):
//   1. running products along each request's lanes: step t hands the
//      products one lane to the right (DPP wave shift) and lane i = t
//      multiplies by its own estimate, so every product is formed with the
//      same roundings as one running product over the request;
//   2. a histogram of the candidates' keys by their top 12 bits; a block scan
//      from the top finds the digit holding the B-th largest and how many of
//      its keys are taken;
//   3. that digit's candidates are listed in LDS, and the one whose rank among
//      them (selection key, then position: (s desc, r asc, i asc)) is the
//      remainder minus one is the threshold; a candidate is taken iff its
//      (key, position) order word is at or above the threshold's;
//   4. L_r by ballot over the request's lanes; offsets by a wave scan.
constexpr int kFastDigitBits = 12;                       // first digit: key bits 29..18
constexpr int kFastBins = 1 << kFastDigitBits;
constexpr int kFastShift = 30 - kFastDigitBits;

template <int NT>
__global__ __launch_bounds__(NT) void k_dvl_lanes(const float* __restrict__ a, int R, int b,
                                                 const int32_t* __restrict__ block_len,
                                                 const int32_t* __restrict__ budget, float* __restrict__ s,
                                                 int32_t* __restrict__ L, int32_t* __restrict__ pos_off,
                                                 int32_t* __restrict__ tgt_off, uint32_t* status) {
  constexpr int NW = NT / kWave, kPer = kFastBins / NT;
  static_assert(kPer * NT == kFastBins, "digits must split evenly over the block");
  __shared__ uint32_t hist[kFastBins];
  __shared__ uint64_t listed[NT];
  __shared__ int wtot[NW];
  __shared__ int lens[kWave];
  __shared__ int sh_listed, sh_digit, sh_rem;
  __shared__ uint64_t sh_thr;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
  const int n = R * b;
  const bool in = tid < n;
  const int r = tid / b, i = tid - r * b;
  // every global load issued before any is used
  const float av = in ? a[tid] : 0.0f;
  const int blr = block_len && in ? block_len[r] : b;
  int B = *budget;
  for (int k = tid; k < kFastBins; k += NT) hist[k] = 0u;
  if (tid == 0) sh_listed = 0;
  if (B < 0) {
    if (tid == 0) raise_status(status, SV_ST_BAD_BUDGET);
    B = 0;
  }
  const int br = min(max(blr, 0), b);
  const bool cand = in && i < br;
  if (__ballot(in && i == 0 && block_len && (blr < 0 || blr > b)) && lane == 0) raise_status(status, SV_ST_BAD_BLOCK);
  if (__ballot(cand && !(av >= 0.0f && av <= 1.0f)) && lane == 0) raise_status(status, SV_ST_BAD_SCORE);
  // 1. running products (lanes of one request are consecutive in the wave)
  float run = 1.0f * av;
  for (int t = 1; t < b; ++t) {
    const float left = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(run), 0x138, 0xF, 0xF, false));
    run = i == t ? left * av : run;  // wave_shr:1: lane l reads lane l - 1
  }
  const float score = cand ? run : 0.0f;
  const uint32_t key = cand ? select_key(run) : 0u;
  const uint32_t digit = key >> kFastShift;
  const uint64_t ord = cand ? (static_cast<uint64_t>(key) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(tid)) : 0ull;
  __syncthreads();  // the histogram and the list are cleared
  // 2. histogram of the candidates' first digits, crossing digit from the top
  if (cand) atomicAdd(&hist[digit], 1u);
  __syncthreads();
  int hv[kPer], hs = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    hv[j] = static_cast<int>(hist[kFastBins - 1 - (tid * kPer + j)]);
    hs += hv[j];
  }
  const int inc = wave_incl_scan_i32(hs);
  if (lane == kWave - 1) wtot[wv] = inc;
  __syncthreads();
  int base = 0, ncand = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    base += k < wv ? wtot[k] : 0;
    ncand += wtot[k];
  }
  const bool all = B >= ncand, none = B == 0;
  const int excl = base + inc - hs;
  if (!all && !none && excl < B && B <= excl + hs) {
    int run_c = excl;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (run_c < B && B <= run_c + hv[j]) {
        sh_digit = kFastBins - 1 - (tid * kPer + j);
        sh_rem = B - run_c;
      }
      run_c += hv[j];
    }
  }
  __syncthreads();
  // 3. the threshold among the crossing digit's candidates
  uint64_t thr = 0;
  if (!all && !none) {
    const bool mine = cand && digit == static_cast<uint32_t>(sh_digit);
    if (mine) listed[atomicAdd(&sh_listed, 1)] = ord;
    __syncthreads();
    const int m = sh_listed, rem = sh_rem;
    if (mine) {
      int rank = 0;
      for (int k = 0; k < m; ++k) rank += listed[k] > ord ? 1 : 0;
      if (rank == rem - 1) sh_thr = ord;
    }
    __syncthreads();
    thr = sh_thr;
  }
  const bool take = cand && (all || (!none && ord >= thr));
  // 4. L_r by ballot over the request's lanes, then the offsets
  const uint64_t tk = __ballot(take);
  if (in && i == 0) {
    const uint64_t seg = b == kWave ? ~0ull : ((1ull << b) - 1ull) << lane;
    lens[r] = __popcll(tk & seg);
  }
  __syncthreads();
  if (wv == 0) {
    const int Lr = lane < R ? lens[lane] : 0;
    const int incl = wave_incl_scan_i32(Lr);
    if (lane < R) {
      L[lane] = Lr;
      pos_off[lane] = incl - Lr;
      tgt_off[lane] = incl - Lr + lane;
    }
    if (lane == R - 1) {
      pos_off[R] = incl;
      tgt_off[R] = incl + R;
    }
  }
  if (in) s[tid] = score;
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
  const int n = R * b;
  if ((b & (b - 1)) == 0 && R <= kWave && n <= 1024) {  // b divides 64: the short-block path
    uint32_t* stw = status_word(ws);
    if (n <= 256)
      hipLaunchKernelGGL(k_dvl_lanes<256>, dim3(1), dim3(256), 0, st, a, R, b, block_len, budget, s, L, pos_off,
                         tgt_off, stw);
    else if (n <= 512)
      hipLaunchKernelGGL(k_dvl_lanes<512>, dim3(1), dim3(512), 0, st, a, R, b, block_len, budget, s, L, pos_off,
                         tgt_off, stw);
    else
      hipLaunchKernelGGL(k_dvl_lanes<1024>, dim3(1), dim3(1024), 0, st, a, R, b, block_len, budget, s, L, pos_off,
                         tgt_off, stw);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
  }
  if (R * b <= kDvlLds)
    hipLaunchKernelGGL(k_dvl<true>, dim3(1), dim3(kDvlNT), 0, st, a, R, b, block_len, budget, s, L, pos_off,
                       tgt_off, status_word(ws));
  else
    hipLaunchKernelGGL(k_dvl<false>, dim3(1), dim3(kDvlNT), 0, st, a, R, b, block_len, budget, s, L, pos_off,
                       tgt_off, status_word(ws));
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}
