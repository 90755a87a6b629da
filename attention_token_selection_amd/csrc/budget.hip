// Kept importance of a budget ("KVDrive: A Holistic Multi-Tier KV Cache
// Management System for Long-Context LLM Inference", §5.2, as the benefit
// of a (layer, head) pair's size): the sum of the pooled scores at the
// positions a top-k selection kept.  One workgroup per (sequence, KV head)
// segment; each thread sums every 256th kept entry in order and the 256
// partial sums are combined in a fixed tree, so the result is reproducible.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void mass_kernel(MassParams p, SegTable t) {
  __shared__ float part[NT];
  const int segl = blockIdx.x;  // local segment: sequence-major, head-minor
  const int sb = segl / p.Hkv;
  const int h = segl - sb * p.Hkv;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  const float *P = p.pooled + (int64_t)p.Hkv * key0 + (int64_t)h * L;
  const int32_t *idx = p.idx + t.out_off[segl];
  const int n = t.keff[segl];
  float s = 0.0f;
  for (int j = threadIdx.x; j < n; j += NT) {
    const int pos = idx[j];
    s += ((unsigned)pos < (unsigned)L) ? P[pos] : 0.0f;
  }
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.mass[(int64_t)(t.seg0 + segl) * p.n_sizes + p.j] = part[0];
}

}  // namespace

hipError_t launch_mass(const MassParams &p, const SegTable &t, hipStream_t s) {
  const int nseg = t.nseq * p.Hkv;
  if (nseg <= 0) return hipSuccess;
  hipLaunchKernelGGL(mass_kernel, dim3(nseg), dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel
