// Mean query per KV-head group: the DeferKV guide's grouped-query shortcut
// ("DeferKV Guide: Eviction Timing for KV Cache Compression", Phase 2 code)
// averages the G query heads of each group before the product with the keys.
// The mean of bf16 queries is formed exactly (a sum of G bf16 values in fp64,
// one division) and rounded once to the nearest bf16 value, ties to even, so
// the score kernels then see one bf16 query row per observation row.
//
// Each 16-lane group handles one (sequence, row, KV head): lane j covers
// components 8j .. 8j+7 with one 16-byte load per query head.
#include <cmath>

#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kItemsPerBlock = 16;

__device__ inline double bf16_lo(uint32_t w) { return (double)__uint_as_float(w << 16); }
__device__ inline double bf16_hi(uint32_t w) { return (double)__uint_as_float(w & 0xffff0000u); }

// Nearest bf16 value, ties to even.  bf16 keeps 8 significant bits, so the
// spacing at |x| in [2^(e-1), 2^e) is 2^(e-8), and never below 2^-133 (the
// subnormal spacing).  The result has at most 8 significant bits, so it is
// exact in fp32, whose upper half is then the bf16 bit pattern.
__device__ inline uint32_t to_bf16_rne(double x) {
  if (x == 0.0) return 0u;
  int e;
  (void)frexp(x, &e);
  const int q = max(e - 8, -133);
  const double y = ldexp(rint(ldexp(x, -q)), q);
  return __float_as_uint((float)y) >> 16;
}

__global__ __launch_bounds__(256) void query_mean_kernel(QueryMeanParams p) {
  const int item = blockIdx.x * kItemsPerBlock + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  if (item >= p.items) return;
  const int h = item % p.Hkv;
  const int64_t br = item / p.Hkv;  // sequence * w' + row
  const uint4 *src = p.Q + (br * p.Hq + (int64_t)h * p.G) * 16 + part;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int g = 0; g < p.G; ++g) {
    const uint4 v = src[(int64_t)g * 16];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += bf16_lo(w[j]);
      acc[2 * j + 1] += bf16_hi(w[j]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = to_bf16_rne(acc[2 * j] / p.G) | (to_bf16_rne(acc[2 * j + 1] / p.G) << 16);
  p.Qm[(int64_t)item * 16 + part] = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_query_mean(const QueryMeanParams &p, hipStream_t s) {
  if (p.items <= 0) return hipSuccess;
  const int blocks = (p.items + kItemsPerBlock - 1) / kItemsPerBlock;
  hipLaunchKernelGGL(query_mean_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace kvsel
