// sv_device.hpp -- device helpers shared by the libsv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv.h"

namespace sv {

constexpr int kWave = 64;

// ------------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): ten rounds; each round multiplies words 0 and 2 by two odd 32-bit
// constants, mixes the high halves with words 1, 3 and the key, and the key
// advances by two Weyl increments between rounds.
struct U4 {
  uint32_t x, y, z, w;
};

__host__ __device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                     uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t pa = static_cast<uint64_t>(kMulA) * c0;  // v_mul_hi_u32 / v_mul_lo_u32 on the GPU
    const uint64_t pb = static_cast<uint64_t>(kMulB) * c2;
    const uint32_t hiA = static_cast<uint32_t>(pa >> 32), loA = static_cast<uint32_t>(pa);
    const uint32_t hiB = static_cast<uint32_t>(pb >> 32), loB = static_cast<uint32_t>(pb);
    const uint32_t n0 = hiB ^ c1 ^ k0;
    const uint32_t n2 = hiA ^ c3 ^ k1;
    c0 = n0;
    c1 = loB;
    c2 = n2;
    c3 = loA;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return U4{c0, c1, c2, c3};
}

// Words at counter (pos, req, 0, 0) under key = 64-bit seed.
__device__ __forceinline__ U4 philox_at(uint64_t seed, uint32_t pos, uint32_t req) {
  return philox4x32_10(pos, req, 0u, 0u, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

// 24-bit uniform on {0, 2^-24, ..., 1 - 2^-24}; exact in float and double.
__device__ __forceinline__ double u24(uint32_t w) { return static_cast<double>(w >> 8) * (1.0 / 16777216.0); }

// ------------------------------------------------------------------ values
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int DT>
__device__ __forceinline__ float load_val(const void* base, int64_t idx) {
  if constexpr (DT == SV_BF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

__device__ __forceinline__ float load_val_rt(const void* base, int dtype, int64_t idx) {
  return dtype == SV_BF16 ? load_val<SV_BF16>(base, idx) : load_val<SV_F32>(base, idx);
}

// Streaming 16-byte load (the data is read once).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_stream(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}

// ------------------------------------------------------------------ wave reductions
// Cross-lane steps use DPP (quad permutes, row mirrors and row shifts inside
// 16-lane rows) and v_readlane for the four row results, so no step takes an
// LDS round trip.  Every caller runs them with all 64 lanes of the wave active;
// the `lane` argument of the broadcasts is wave-uniform.
namespace dpp {
constexpr int kXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int kMirror = 0x140;      // lane i <- 15 - i within each row
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;  // row_shr:n (0 shifted in)
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(dpp_i32<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  return __hiloint2double(dpp_i32<CTRL>(__double2hiint(v)), dpp_i32<CTRL>(__double2loint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(dpp_i32<CTRL>(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(dpp_i32<CTRL>(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ int bcast_i32(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float bcast_f32(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ double bcast_f64(double v, int lane) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), lane),
                          __builtin_amdgcn_readlane(__double2loint(v), lane));
}
__device__ __forceinline__ uint64_t bcast_u64(uint64_t v, int lane) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), lane));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), lane));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Butterfly inside each row (every lane of a row ends with the row's result:
// each step combines the same two operands in either order), then the four
// row results in a fixed order.  Identical in every lane.
#define SV_WAVE_REDUCE(T, SUF, OP)                                                  \
  v = OP(v, dpp_##SUF<dpp::kXor1>(v));                                              \
  v = OP(v, dpp_##SUF<dpp::kXor2>(v));                                              \
  v = OP(v, dpp_##SUF<dpp::kHalfMirror>(v));                                        \
  v = OP(v, dpp_##SUF<dpp::kMirror>(v));                                            \
  return OP(OP(bcast_##SUF(v, 0), bcast_##SUF(v, 16)), OP(bcast_##SUF(v, 32), bcast_##SUF(v, 48)))

__device__ __forceinline__ double sv_add_f64(double a, double b) { return a + b; }
__device__ __forceinline__ uint64_t sv_max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ int sv_min_i32(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int sv_max_i32(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) { SV_WAVE_REDUCE(uint64_t, u64, sv_max_u64); }
__device__ __forceinline__ double wave_sum_f64(double v) { SV_WAVE_REDUCE(double, f64, sv_add_f64); }
__device__ __forceinline__ int wave_min_i32(int v) { SV_WAVE_REDUCE(int, i32, sv_min_i32); }
__device__ __forceinline__ int wave_max_i32(int v) { SV_WAVE_REDUCE(int, i32, sv_max_i32); }
__device__ __forceinline__ float wave_max_f32(float v) { SV_WAVE_REDUCE(float, f32, fmaxf); }
#undef SV_WAVE_REDUCE

// Inclusive scan over the wave in lane order: shifts by 1, 2, 4, 8 inside each
// row, then the totals of the rows before.
__device__ __forceinline__ double wave_incl_scan_f64(double v) {
  const int row = (threadIdx.x & (kWave - 1)) >> 4;
  v += dpp_f64<dpp::kShr1>(v);
  v += dpp_f64<dpp::kShr2>(v);
  v += dpp_f64<dpp::kShr4>(v);
  v += dpp_f64<dpp::kShr8>(v);
  const double r0 = bcast_f64(v, 15), r1 = bcast_f64(v, 31), r2 = bcast_f64(v, 47);
  const double r01 = r0 + r1;
  const double off = row == 0 ? 0.0 : row == 1 ? r0 : row == 2 ? r01 : r01 + r2;
  return off + v;
}

__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  const int row = (threadIdx.x & (kWave - 1)) >> 4;
  v += dpp_i32<dpp::kShr1>(v);
  v += dpp_i32<dpp::kShr2>(v);
  v += dpp_i32<dpp::kShr4>(v);
  v += dpp_i32<dpp::kShr8>(v);
  const int r0 = bcast_i32(v, 15), r1 = bcast_i32(v, 31), r2 = bcast_i32(v, 47);
  const int off = row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2;
  return off + v;
}

// ------------------------------------------------------------------ block reductions
// All threads of the block must call these.  `scratch` holds >= NT/64 items.
template <int NT>
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* scratch) {
  constexpr int NW = NT / kWave;
  v = wave_max_u64(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  uint64_t r = scratch[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) r = scratch[k] > r ? scratch[k] : r;
  return r;
}

template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* scratch) {
  constexpr int NW = NT / kWave;
  v = wave_sum_f64(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int k = 0; k < NW; ++k) r += scratch[k];  // fixed order: deterministic
  return r;
}

template <int NT>
__device__ __forceinline__ int block_min_i32(int v, int* scratch) {
  constexpr int NW = NT / kWave;
  v = wave_min_i32(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  int r = scratch[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) r = scratch[k] < r ? scratch[k] : r;
  return r;
}

// Exclusive scan in thread order; also returns the block total.
template <int NT>
__device__ __forceinline__ double block_excl_scan_f64(double v, double* scratch, double* total) {
  constexpr int NW = NT / kWave;
  const double inc = wave_incl_scan_f64(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == kWave - 1) scratch[w] = inc;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (k < w) base += scratch[k];
    tot += scratch[k];
  }
  *total = tot;
  return base + inc - v;
}

template <int NT>
__device__ __forceinline__ int block_excl_scan_i32(int v, int* scratch, int* total) {
  constexpr int NW = NT / kWave;
  const int inc = wave_incl_scan_i32(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == kWave - 1) scratch[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    if (k < w) base += scratch[k];
    tot += scratch[k];
  }
  *total = tot;
  return base + inc - v;
}

// ------------------------------------------------------------------ ragged offsets
// Request r with off[r] <= p < off[r+1]; -1 if none (malformed offsets).
// All threads of the block must call this; `slot` is one shared int.
template <int NT>
__device__ __forceinline__ int find_request(const int32_t* off, int R, int p, int* slot) {
  if (threadIdx.x == 0) *slot = -1;
  __syncthreads();
  for (int r = threadIdx.x; r < R; r += NT) {
    if (off[r] <= p && p < off[r + 1]) *slot = r;
  }
  __syncthreads();
  return *slot;
}

// ------------------------------------------------------------------ status
__device__ __forceinline__ void raise_status(uint32_t* status, uint32_t bits) {
  __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ exp in double
// exp(x) by Tang's table method (P. T. P. Tang, "Table-driven implementation
// of the exponential function in IEEE floating-point arithmetic", ACM TOMS 15,
// 1989): x = (64 k + j) ln2/64 + r with |r| <= ln2/128, so that
// exp(x) = 2^k 2^(j/64) e^r; e^r by its Taylor polynomial of degree 5 (the
// first omitted term is below 4e-17 relative), 2^(j/64) from a 64-entry table
// in LDS (exp_table_init), 2^k by ldexp, which rounds once and underflows
// gradually.  ln2/64 is split into a 36-bit head (k times it is exact for
// |k| < 2^17) and the rounded remainder.  Meant for the arguments of the
// probabilities (x <= 0 up to rounding); x < -746 gives 0 and NaN stays NaN.
constexpr int kExpTab = 64;

// tab[t] = 2^(t/64), by threads 0..63 of the block; the caller's next barrier
// publishes it.
__device__ __forceinline__ void exp_table_init(double* tab) {
  const int t = threadIdx.x;
  if (t < kExpTab) tab[t] = exp2(static_cast<double>(t) / kExpTab);
}

__device__ __forceinline__ double exp_tab(double x, const double* tab) {
  constexpr double kInvStep = 0x1.71547652b82fep+6;    // 64 / ln 2
  constexpr double kStepHi = 0x1.62e42fefa0000p-7;     // ln 2 / 64, 36 significant bits
  constexpr double kStepLo = 0x1.cf79abc9e3b3ap-46;    // ln 2 / 64 - kStepHi
  const double xc = x > -746.0 ? x : -746.0;           // NaN and -inf handled at the end
  const double kd = __builtin_rint(xc * kInvStep);
  const int k = static_cast<int>(kd);
  double r = fma(-kd, kStepHi, xc);
  r = fma(-kd, kStepLo, r);
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  const double y = ldexp(tab[k & (kExpTab - 1)] * p, k >> 6);
  return x > -746.0 ? y : (x != x ? x : 0.0);
}

// ------------------------------------------------------------------ the draw's row layout
// The row a request draws from is cut into sub-chunks of 64 8-value groups
// (512 values, one group per lane of a wave); one block of the sums kernel
// (kSumNT threads) covers a chunk of kSubPerWave sub-chunks per wave.
constexpr int kSumNT = 256;
constexpr int kSubG = 64;
constexpr int kSubPerWave = 2;
constexpr int kChunkSubs = kSubPerWave * (kSumNT / kWave);  // 8 sub-chunks, 512 groups (a block per 4096 values)

__host__ __device__ inline int groups_of(int V) { return (V + 7) / 8; }
__host__ __device__ inline int sub_chunks(int V) { return (groups_of(V) + kSubG - 1) / kSubG; }
__host__ __device__ inline int res_chunks(int V) { return (sub_chunks(V) + kChunkSubs - 1) / kChunkSubs; }

// What the draw of one request needs: written by the first chunk block of the
// sums kernel, read by the pick kernel.
// kDrawResidual: norm(max(0, p - q)) with q a dense draft row or the point
// masses of greedy branches (corrections at their tokens); kDrawSoft: q the
// posterior-weighted sum of K soft branch rows; kDrawP: p (bonus, or T = 0
// fallback); kDrawGreedy: the argmax; kDrawNone: malformed offsets.
enum : int32_t { kDrawResidual = 0, kDrawP = 1, kDrawGreedy = 2, kDrawNone = 3, kDrawSoft = 4 };
struct DrawRec {
  int32_t mode, n, bonus, token;  // token: the argmax when greedy
  int32_t ncorr, pad0;
  int64_t trow, drow;  // target row of the draw; dense draft row, or branch 0's row (soft)
  float cut, pad1;
  double invT, kept, dlse;
  double invTb;      // soft branches: 1 / T_b
  int32_t ctok[64];  // greedy-branch residual: the distinct branch tokens at the slot
  double cw[64];     // soft: lse_z - log w_z per branch z
  double cq[64];     // greedy-branch residual: q at those tokens (the summed weights of
                     // the branches on each); the draw weight there is max(0, p - q)
};

// What the fused rows launches leave for the draw, per request r and target row
// j <= L_r, at slot r * (b + 1) + j: the row's statistics and, for j < L_r,
// the target logit at draft token j (as fp32), so that the draw reads them by
// request and position without first reading the row offsets.  The dense
// draft's row for position j has a slot of its own (kept = its lse, argmax,
// lx = its logit at the draft token).
struct SlotRec {
  double kept;
  float cut;
  int32_t argmax;
  float lx;
  int32_t pad;
};

// ------------------------------------------------------------------ branch argmax parts
// In the fused rows launch each component row is streamed by kMixParts blocks
// (contiguous quarters of its 16-byte vectors); each writes its partial
// argmax as a packed key (order key of the value above the complemented
// index, 0 if it saw nothing) to its own workspace slot, and the draw's first
// load round takes the largest key of the parts.
constexpr int kMixParts = 4;

__device__ __host__ inline uint32_t argmax_token(uint64_t key) {
  return key ? 0xFFFFFFFFu - static_cast<uint32_t>(key) : 0u;
}

// ------------------------------------------------------------------ split rows
// sv_verify_rows_dense streams each row without a top-p cut as P blocks
// (contiguous parts of its vectors; P = kRowParts when a top-p value is given,
// else up to kDenseMaxParts); each leaves its partial statistics in the
// workspace and a second launch merges them.  Part 0 of every row also
// records whether the row was split (rows with a cut, and fp32 rows, are done
// whole by part 0).
constexpr int kRowParts = 2;
constexpr int kDenseMaxParts = 16;
struct RowPart {
  double S;      // sum over the part of exp2((l - M) * c2), c2 = log2(e) / T in fp32
  uint64_t key;  // packed argmax key of the part (0: empty)
  float M;       // maximum of the part
  float T;       // the row's temperature
  int32_t split; // part 0: 1 if the row was split, 0 if it was done whole
  int32_t pad;
};

// ------------------------------------------------------------------ workspace layout
// [status word, 256 B][draw records, R][sub-chunk sums, R * NSUB * 2 doubles]
// [branch argmax parts, R * K * b * kMixParts keys]
// [soft branch rows, R * K * b each: lse (double), argmax (int32), max (float)]
// [split-row parts, (R * (b + 1) + R * b) * kDenseMaxParts RowPart records]
// [split-row arrival counts, R * (b + 1) + R * b; zero between launches]
// Cross-block results travel through kernel boundaries (stream order), not
// through in-kernel fences: a device-scope release on gfx950 writes back the
// L2, which is far too costly to pay once per block.
struct WsLayout {
  size_t status, rec, sub, bkey, blse, barg, bmax, rpart, rcount, slot, dslot, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

__host__ __device__ inline WsLayout ws_layout(int R, int b, int K, int V) {
  WsLayout l;
  l.status = 0;
  l.rec = 256;
  l.sub = l.rec + align256(sizeof(DrawRec) * static_cast<size_t>(R));
  l.bkey = l.sub + align256(sizeof(double) * 2 * static_cast<size_t>(R) * sub_chunks(V));
  const size_t kb = static_cast<size_t>(R) * K * b;
  l.blse = l.bkey + align256(sizeof(uint64_t) * kb * kMixParts);
  l.barg = l.blse + align256(sizeof(double) * kb);
  l.bmax = l.barg + align256(sizeof(int32_t) * kb);
  l.rpart = l.bmax + align256(sizeof(float) * kb);
  l.rcount = l.rpart + align256(sizeof(RowPart) * static_cast<size_t>(R) * (2 * b + 1) * kDenseMaxParts);
  l.slot = l.rcount + align256(sizeof(uint32_t) * static_cast<size_t>(R) * (2 * b + 1));
  l.dslot = l.slot + align256(sizeof(SlotRec) * static_cast<size_t>(R) * (b + 1));
  l.total = l.dslot + align256(sizeof(SlotRec) * static_cast<size_t>(R) * (b + 1));
  return l;
}

}  // namespace sv
