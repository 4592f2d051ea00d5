// sv_abi.hip -- workspace, status word and Philox test export of libsv.
#include "sv_device.hpp"
#include "sv_host.hpp"

namespace sv {

__global__ void k_fill_u32(uint32_t* p, size_t n, uint32_t v) {
  for (size_t k = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; k < n;
       k += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[k] = v;
}

__global__ void k_philox(const uint64_t* seed, int R, int n_pos, uint32_t* out) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= R * n_pos) return;
  const int r = k / n_pos, i = k % n_pos;
  const U4 w = philox_at(*seed, static_cast<uint32_t>(i), static_cast<uint32_t>(r));
  uint32_t* o = out + static_cast<size_t>(k) * 4;
  o[0] = w.x;
  o[1] = w.y;
  o[2] = w.z;
  o[3] = w.w;
}

__global__ void k_exp_selftest(const double* x, double* out, int n) {
  __shared__ double tab[kExpTab];
  exp_table_init(tab);
  __syncthreads();
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) out[k] = exp_tab(x[k], tab);
}

}  // namespace sv

using namespace sv;

extern "C" int32_t sv_selftest_exp(const double* x, double* out, int32_t n, void* stream) {
  if (!x || !out || n < 1) return SV_ERR_ARG;
  hipLaunchKernelGGL(k_exp_selftest, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), x, out, n);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_workspace_bytes(int32_t R, int32_t b, int32_t K, int32_t V, size_t* out_bytes) {
  if (!out_bytes || R < 1 || b < 1 || b > 64 || K < 0 || K > 64 || V < 1) return SV_ERR_ARG;
  *out_bytes = ws_layout(R, b, K, V).total;
  return SV_OK;
}

extern "C" int32_t sv_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes < 256 || ws_bytes % 4 != 0) return SV_ERR_ARG;
  const size_t n = ws_bytes / 4;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(ws), n, 0u);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_clear_status(void* ws, void* stream) {
  if (!ws) return SV_ERR_ARG;
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), status_word(ws), size_t{1}, 0u);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" int32_t sv_get_status(const void* ws, void* stream, uint32_t* host_out) {
  if (!ws || !host_out) return SV_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host_out, ws, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return SV_ERR_LAUNCH;
  return hipStreamSynchronize(s) == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

extern "C" const char* sv_status_string(int32_t code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_ERR_ARG: return "invalid argument (null pointer, size out of range, misalignment, dtype or mode)";
    case SV_ERR_WORKSPACE: return "workspace too small";
    case SV_ERR_LAUNCH: return "HIP launch or copy failed";
    case SV_ERR_TOO_LARGE:
      return "problem too large for the fixed scratch of the allocation-free entry point (SV_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status code";
  }
}

extern "C" int32_t sv_philox_uniforms(const uint64_t* seed, int32_t R, int32_t n_pos, uint32_t* out, void* stream) {
  if (!seed || !out || R < 1 || n_pos < 1 || static_cast<long long>(R) * n_pos > 0x7FFFFFFF) return SV_ERR_ARG;
  const int n = R * n_pos;
  hipLaunchKernelGGL(k_philox, dim3((n + 255) / 256), dim3(256), 0, static_cast<hipStream_t>(stream), seed, R, n_pos, out);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

// Host-side self-check of the Philox round function as compiled into this
// library (runs on the CPU; the known-answer vectors of the Random123
// distribution for Philox4x32-10).
extern "C" int32_t sv_selftest_philox_host(void) {
  struct Kat {
    uint32_t c[4], k[2], o[4];
  };
  const Kat kat[3] = {
      {{0, 0, 0, 0}, {0, 0}, {0x6627e8d5u, 0xe169c58du, 0xbc57ac4cu, 0x9b00dbd8u}},
      {{~0u, ~0u, ~0u, ~0u}, {~0u, ~0u}, {0x408f276du, 0x41c83b0eu, 0xa20bc7c6u, 0x6d5451fdu}},
      {{0x243f6a88u, 0x85a308d3u, 0x13198a2eu, 0x03707344u}, {0xa4093822u, 0x299f31d0u},
       {0xd16cfe09u, 0x94fdccebu, 0x5001e420u, 0x24126ea1u}},
  };
  for (int t = 0; t < 3; ++t) {
    const U4 w = philox4x32_10(kat[t].c[0], kat[t].c[1], kat[t].c[2], kat[t].c[3], kat[t].k[0], kat[t].k[1]);
    if (w.x != kat[t].o[0] || w.y != kat[t].o[1] || w.z != kat[t].o[2] || w.w != kat[t].o[3]) return t + 1;
  }
  return 0;
}
