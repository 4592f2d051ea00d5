// sv_rows.hip -- entry points for per-row statistics (see sv_rows_dev.hpp for
// the method): sv_softmax_stats and sv_topp_threshold, one block per row.
#include "sv_host.hpp"
#include "sv_rows_dev.hpp"

namespace sv {

constexpr int kRowNT = 512;
constexpr int kRowBatch = 4;  // 16-byte loads per thread per batch (x2 in flight): 114 VGPRs, two blocks per CU
constexpr int kDenseNT = 256;  // sv_verify_rows_dense: P blocks of 256 per split row
constexpr int kDenseBatch = 4;
constexpr int kDensePartVec = 6400;  // vectors per part (100 KiB of bf16) without a cut

// Row p of a's rows (p < the device-side count), by one block.
template <int DT>
__device__ __forceinline__ void stats_block(const RowArgs& a, int p, uint32_t* hist, RowShared<kRowNT>& sh) {
  const int total = a.row_off[a.R];
  if (p == 0 && threadIdx.x == 0 && (a.row_off[0] != 0 || total > a.max_rows || total < 0))
    raise_status(a.status, SV_ST_BAD_OFFSETS);
  if (p >= total) return;
  exp_table_init(sh.etab);  // published by row_block's first barrier
  row_block<DT, kRowNT, kRowBatch>(a, p, hist, sh);
}

template <int DT>
__global__ __launch_bounds__(kRowNT) void k_row_stats(RowArgs a) {
  __shared__ RowShared<kRowNT> sh;
  __shared__ uint32_t hist[DT == SV_BF16 ? kHistWords : 1];
  stats_block<DT>(a, blockIdx.x, hist, sh);
}

// A part record through agent-scope atomics: the parts of a row are written
// and read by different blocks of one launch, which may sit on different
// compute dies (the stores reach the device-coherent level; the loads read it).
__device__ __forceinline__ void store_part(RowPart* dst, const RowPart& o) {
  static_assert(sizeof(RowPart) == 32, "a part record is four 8-byte words");
  const uint64_t* w = reinterpret_cast<const uint64_t*>(&o);
  uint64_t* d = reinterpret_cast<uint64_t*>(dst);
#pragma unroll
  for (int k = 0; k < 4; ++k) __hip_atomic_store(d + k, w[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The row's statistics from its P parts, by one wave (lane k < P reads part
// k's record with agent-scope atomic loads): maximum and argmax key by max,
// the sums rescaled to the row maximum in double with the parts' own scale
// constant, lse = M / T + log(S).
__device__ __forceinline__ void merge_parts_wave(const RowArgs& a, int p, int P, const RowPart* rec) {
  const int lane = threadIdx.x & (kWave - 1);
  uint64_t w[4] = {0, 0, 0, 0};
  if (lane < P)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = __hip_atomic_load(reinterpret_cast<const uint64_t*>(rec + lane) + j, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
  RowPart r;
  __builtin_memcpy(&r, w, sizeof(RowPart));
  const float Mk = lane < P ? r.M : -INFINITY;
  const float M = wave_max_f32(Mk);
  const uint64_t key = wave_max_u64(lane < P ? r.key : 0ull);
  const float T = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r.T)));  // lane 0: part 0
  const int am = static_cast<int>(argmax_token(key));
  if (T == 0.0f) {
    if (lane == 0) write_row(a, p, M, am, 0.0, M, 0.0);
    return;
  }
  const double c2 = static_cast<double>(soft_c2(T));
  const double term = Mk > -INFINITY ? r.S * exp2((static_cast<double>(Mk) - static_cast<double>(M)) * c2) : 0.0;
  const double S = wave_sum_f64(term);
  if (lane == 0) {
    const double lse = static_cast<double>(M) / static_cast<double>(T) + log(S);
    write_row(a, p, M, am, lse, -INFINITY, lse);
  }
}

// Part `part` of row p of a (sv_verify_rows_dense).  A bf16 row without a
// top-p cut is streamed as P blocks, each leaving its partial statistics in
// parts[p * P + part] and counting itself in count[p]; the block that arrives
// last merges the parts and writes the row (and sets count[p] back to 0).  Any
// other row is done whole by part 0, which marks it unsplit.  kCut = false: no
// row of a has a top-p value (a.top_p is null), so the cut's histogram code,
// table and LDS are left out.
template <int DT, int NT, int BATCH, bool kCut>
__device__ __forceinline__ void stats_part(const RowArgs& a, int p, int part, int P, RowPart* parts, uint32_t* count,
                                           uint32_t* hist, RowShared<NT>& sh) {
  const int total = a.row_off[a.R];
  if (p == 0 && part == 0 && threadIdx.x == 0 && (a.row_off[0] != 0 || total > a.max_rows || total < 0))
    raise_status(a.status, SV_ST_BAD_OFFSETS);
  if (p >= total) return;
  if (kCut) exp_table_init(sh.etab);  // published by row_locate's barriers
  const RowLoc l = row_locate<DT, NT>(a, p, sh);
  if (!l.ok) return;
  const RowArgs s = with_slot(a, l);  // the row's slot record goes with its statistics
  RowPart* rec = parts + static_cast<size_t>(p) * P;
  const bool topp_on = kCut && l.topp_on;
  if (DT != SV_BF16 || topp_on) {
    if (part != 0) return;
    row_stats_at<DT, NT, BATCH>(s, l.rowp, p, l.T, l.tp, topp_on, hist, sh);
    if (threadIdx.x == 0) rec[0].split = 0;
    if (threadIdx.x == NT - 1) slot_gather<DT>(s, l);
    return;
  }
  const int nvec = a.V >> 3;
  const int v0 = static_cast<int>(static_cast<int64_t>(nvec) * part / P);
  const int v1 = static_cast<int>(static_cast<int64_t>(nvec) * (part + 1) / P);
  const StreamPart sp = stream_part_bf16<NT, BATCH>(static_cast<const uint16_t*>(l.rowp), a.V, v0, v1, part == P - 1,
                                                     l.T, a.status, sh);
  if (part == 0 && threadIdx.x == NT - 1) slot_gather<DT>(s, l);  // a wave that is otherwise done
  if (threadIdx.x < kWave) {  // wave 0
    uint32_t arrived = 0;
    if (threadIdx.x == 0) {
      RowPart o;
      o.S = sp.S;
      o.key = sp.key;
      o.M = sp.M;
      o.T = l.T;
      o.split = 1;
      o.pad = 0;
      store_part(rec + part, o);
      __builtin_amdgcn_s_waitcnt(0);  // the record is at the device-coherent level before the part counts itself in
      arrived = __hip_atomic_fetch_add(count + p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (__builtin_amdgcn_readfirstlane(arrived) == static_cast<uint32_t>(P - 1)) {  // the row's last part
      if (threadIdx.x == 0) __hip_atomic_store(count + p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      merge_parts_wave(s, p, P, rec);
    }
  }
}

// The packed target rows and the dense draft's rows in one grid
// (sv_verify_rows_dense): P blocks per row, target rows first, then draft
// rows; blocks past a row set's device-side count exit after the lookup.
// Many short blocks let the dispatcher keep every compute unit streaming to
// the end (a compute unit issues its oldest waves first, so equal shares of
// long blocks would end at unequal times).  Draft rows never take a cut;
// kCut is false when no target row can either.
template <int DT, int DDT, bool kCut>
__global__ __launch_bounds__(kDenseNT) void k_rows_dense(RowArgs ta, RowArgs da, int n_tgt, int P, RowPart* tparts,
                                                         RowPart* dparts, uint32_t* tcount, uint32_t* dcount) {
  __shared__ RowShared<kDenseNT> sh;
  __shared__ uint32_t hist[kCut && DT == SV_BF16 ? kHistWords : 1];
  const int q = blockIdx.x / P, part = blockIdx.x % P;
  if (q < n_tgt)
    stats_part<DT, kDenseNT, kDenseBatch, kCut>(ta, q, part, P, tparts, tcount, hist, sh);
  else
    stats_part<DDT, kDenseNT, kDenseBatch, false>(da, q - n_tgt, part, P, dparts, dcount, hist, sh);
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

// Host-side self-check of the pure helpers in sv_rows_dev.hpp (runs on the CPU).
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

// The cut's histogram (and its LDS, table and registers) only where a top-p value is given.
template <int DT, int DDT>
static int32_t launch_dense(const RowArgs& ta, const RowArgs& da, int32_t n_tgt, int P, RowPart* tparts,
                            RowPart* dparts, uint32_t* tcount, uint32_t* dcount, unsigned grid, hipStream_t s) {
  if (ta.top_p)
    hipLaunchKernelGGL((k_rows_dense<DT, DDT, true>), dim3(grid), dim3(kDenseNT), 0, s, ta, da, n_tgt, P, tparts,
                       dparts, tcount, dcount);
  else
    hipLaunchKernelGGL((k_rows_dense<DT, DDT, false>), dim3(grid), dim3(kDenseNT), 0, s, ta, da, n_tgt, P, tparts,
                       dparts, tcount, dcount);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_verify_rows_dense(const void* tgt_logits, int32_t dtype, int64_t tgt_ld, int32_t V,
                                        const int32_t* tgt_off, int32_t R, int32_t max_rows,
                                        const float* temperature, const float* top_p, float* row_max,
                                        int32_t* row_argmax, double* row_lse, float* row_cut,
                                        double* row_kept_lse, const void* draft_logits, int32_t draft_dtype,
                                        int64_t draft_ld, int32_t b, const int32_t* pos_off, int32_t max_pos,
                                        const int32_t* draft_tok, float* draft_max, int32_t* draft_argmax,
                                        double* draft_lse, void* ws, size_t ws_bytes, void* stream) {
  if (!tgt_logits || !tgt_off || !temperature || !row_max || !row_argmax || !row_lse || !row_cut || !row_kept_lse)
    return SV_ERR_ARG;
  if (!draft_logits || !pos_off || !draft_tok || !draft_max || !draft_argmax || !draft_lse || !ws) return SV_ERR_ARG;
  if (R < 1 || V < 1 || b < 1 || b > 64 || max_rows < 0 || max_pos < 0 || tgt_ld < V || draft_ld < V)
    return SV_ERR_ARG;
  if ((dtype != SV_F32 && dtype != SV_BF16) || (draft_dtype != SV_F32 && draft_dtype != SV_BF16)) return SV_ERR_ARG;
  if (!rows_aligned(tgt_logits, dtype, tgt_ld) || !rows_aligned(draft_logits, draft_dtype, draft_ld)) return SV_ERR_ARG;
  if (static_cast<long long>(max_pos) > static_cast<long long>(R) * b) return SV_ERR_ARG;
  if (static_cast<long long>(max_rows) + max_pos > 0x7FFFFFFFLL) return SV_ERR_ARG;
  if (max_rows > R * (b + 1)) return SV_ERR_ARG;
  const WsLayout l = ws_layout(R, b, 0, V);
  if (ws_bytes < l.total) return SV_ERR_WORKSPACE;
  const unsigned n_all = static_cast<unsigned>(max_rows) + static_cast<unsigned>(max_pos);
  if (n_all == 0) return SV_OK;
  const int nvec = V >> 3;
  int P = kRowParts;  // parts per split row
  if (!top_p) P = nvec >= kDensePartVec * kDenseMaxParts ? kDenseMaxParts : (nvec + kDensePartVec - 1) / kDensePartVec;
  P = P < 1 ? 1 : P;
  if (static_cast<unsigned long long>(n_all) * P > 0x7FFFFFFFull) return SV_ERR_ARG;
  const unsigned grid = n_all * static_cast<unsigned>(P);
  RowPart* tparts = reinterpret_cast<RowPart*>(static_cast<char*>(ws) + l.rpart);
  RowPart* dparts = tparts + static_cast<size_t>(R) * (b + 1) * P;
  uint32_t* tcount = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + l.rcount);
  uint32_t* dcount = tcount + static_cast<size_t>(R) * (b + 1);
  RowArgs ta{tgt_logits, tgt_ld, V, tgt_off, 0, R, max_rows, temperature, top_p, row_max, row_argmax, row_lse,
             row_cut, row_kept_lse, status_word(ws)};
  RowArgs da{draft_logits, draft_ld, V, pos_off, b, R, max_pos, temperature, nullptr, draft_max, draft_argmax,
             draft_lse, nullptr, nullptr, status_word(ws)};
  // slot records for the draw: target rows (statistics, logit at the draft
  // token) and draft rows (lse, argmax and logit at the draft token, in the
  // fields kept, argmax and lx)
  ta.slot = reinterpret_cast<SlotRec*>(static_cast<char*>(ws) + l.slot);
  da.slot = reinterpret_cast<SlotRec*>(static_cast<char*>(ws) + l.dslot);
  ta.gx = da.gx = draft_tok;
  ta.slot_b = da.slot_b = b;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool t16 = dtype == SV_BF16, d16 = draft_dtype == SV_BF16;
  const int32_t st = t16 ? (d16 ? launch_dense<SV_BF16, SV_BF16>(ta, da, max_rows, P, tparts, dparts, tcount, dcount, grid, s)
                                : launch_dense<SV_BF16, SV_F32>(ta, da, max_rows, P, tparts, dparts, tcount, dcount, grid, s))
                         : (d16 ? launch_dense<SV_F32, SV_BF16>(ta, da, max_rows, P, tparts, dparts, tcount, dcount, grid, s)
                                : launch_dense<SV_F32, SV_F32>(ta, da, max_rows, P, tparts, dparts, tcount, dcount, grid, s));
  return st;
}
