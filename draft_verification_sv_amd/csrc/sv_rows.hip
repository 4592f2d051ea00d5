// sv_rows.hip -- entry points for per-row statistics (see sv_rows_dev.hpp for
// the method): sv_softmax_stats and sv_topp_threshold, one block per row.
#include "sv_host.hpp"
#include "sv_rows_dev.hpp"

namespace sv {

constexpr int kRowNT = 512;
constexpr int kRowBatch = 8;  // 16-byte loads per thread per batch (x2 in flight)

template <int DT>
__global__ __launch_bounds__(kRowNT) void k_row_stats(RowArgs a) {
  __shared__ RowShared<kRowNT> sh;
  __shared__ uint32_t hist[DT == SV_BF16 ? kHistWords : 1];
  const int p = blockIdx.x;
  const int total = a.row_off[a.R];
  if (p == 0 && threadIdx.x == 0 && (a.row_off[0] != 0 || total > a.max_rows || total < 0))
    raise_status(a.status, SV_ST_BAD_OFFSETS);
  if (p >= total) return;
  exp_table_init(sh.etab);  // published by row_block's first barrier
  row_block<DT, kRowNT, kRowBatch>(a, p, hist, sh);
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
