// K/V compaction: copy the kept rows of each (sequence, KV head) into the
// flattened variable-length output layout (TideKV §4.1 and §5: retained K/V
// with their original positions, per-head offsets).
//
// A row is d = 128 bf16 = 256 bytes = 16 lanes x 16 bytes, so a 256-thread
// workgroup moves 16 rows of K and 16 rows of V with fully coalesced 16-byte
// loads and stores.  Indices outside the sequence produce zero rows instead
// of reading out of bounds.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kRowsPerBlock = 16;

__global__ __launch_bounds__(256) void gather_kernel(GatherParams p, SegTable t) {
  const int h = blockIdx.y;
  const int sb = blockIdx.z;
  const int segl = sb * p.Hkv + h;
  const int j = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  if (j >= t.keff[segl]) return;
  const int64_t o = t.out_off[segl] + j;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  const int pos = p.idx[o];
  uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
  if ((unsigned)pos < (unsigned)L) {
    const int64_t src = ((key0 + pos) * p.Hkv + h) * 16 + part;
    kv = p.K[src];
    vv = p.V[src];
  }
  p.K_out[o * 16 + part] = kv;
  p.V_out[o * 16 + part] = vv;
}

}  // namespace

hipError_t launch_gather(const GatherParams &p, const SegTable &t, hipStream_t s) {
  if (t.kmax <= 0) return hipSuccess;
  const dim3 grid((t.kmax + kRowsPerBlock - 1) / kRowsPerBlock, p.Hkv, t.nseq);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel
