// Device helpers shared by the selection kernels and pass 2 with tables.
// Included by HIP sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

// The fp32 bits mapped to an unsigned key that orders like the value: a
// larger value has a larger key, and -0 ranks as +0.
__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The key a position competes with: reserved positions (the first `sink`
// and the last `recent` of the sequence; DeferKV guide, Phase 3) take the
// largest key, above every value's, so they are kept first (lowest position
// first among them).
__device__ inline uint32_t select_key(float f, int pos, int L, int sink, int recent) {
  return (pos < sink || pos >= L - recent) ? 0xffffffffu : order_key(f);
}

}  // namespace kvsel
