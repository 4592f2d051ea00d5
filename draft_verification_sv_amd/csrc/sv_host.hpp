// sv_host.hpp -- host-side helpers shared by the libsv entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sv.h"
#include "sv_device.hpp"

namespace sv {

// Base pointer and row pitch of a logit matrix must be 16-byte multiples so
// that every row can be streamed with 128-bit loads.
inline bool rows_aligned(const void* base, int32_t dtype, int64_t ld) {
  const int64_t esz = dtype == SV_BF16 ? 2 : 4;
  return (reinterpret_cast<uintptr_t>(base) % 16 == 0) && ((ld * esz) % 16 == 0);
}

inline uint32_t* status_word(void* ws) { return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + 0); }

}  // namespace sv
