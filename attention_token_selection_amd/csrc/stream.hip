// The selection side of TideKV's memory-bounded streaming top-k ("Delayed KV
// Eviction via Layer-Wise Chunked Prefill", §4.2): the prefix is visited in
// steps of `stream` keys; each step's pooled scores join the running top-k
// in one candidate row per (sequence, KV head), the exact selection kernels
// pick the best k of the row, and the kept slots become the next running
// set.  The running slots hold ascending positions, all before the step's
// keys, so slot order is position order and the selection's tie rule (lower
// slot first) is the whole prefix's (lower position first).  Reserved
// positions (sinks, recent window) enter with +inf, above every score;
// unused slots hold -inf and are never kept (a step keeps at most as many
// slots as hold candidates).
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int NT = 256;

__device__ inline int seq_len(const SegTable &t, int sb) { return (int)(t.key_off[sb + 1] - t.key_off[sb]); }

// Before the first step: no running values yet.
__global__ __launch_bounds__(NT) void stream_init_kernel(StreamParams p, SegTable t) {
  const int seg = t.seg0 + blockIdx.y;
  const int j = blockIdx.x * NT + threadIdx.x;
  if (j < p.kslot) p.cand[(int64_t)seg * p.lv + j] = -INFINITY;
}

// This step's candidates: position i = c0 + x of the segment's sequence,
// pooled from the pass-2 window (zero padded / ignored outside [0, L) as in
// the whole-prefix pool), into slot kslot + x.
__global__ __launch_bounds__(NT) void stream_pool_kernel(StreamParams p, SegTable t) {
  const int sl = blockIdx.y;
  const int sb = sl / p.Hkv;
  const int seg = t.seg0 + sl;
  const int L = seq_len(t, sb);
  const int x = blockIdx.x * NT + threadIdx.x;
  if (x >= p.stream) return;
  const int i = p.c0 + x;
  float v = -INFINITY;
  if (i < L) {
    const float *S = p.S + (int64_t)seg * p.S_stride - p.S_origin;  // S[j] = score of key j
    const int r = (p.pool == 0) ? 0 : (p.pool_kernel - 1) / 2;
    const int a = max(0, i - r), b = min(L - 1, i + r);
    if (p.pool == 2) {
      v = S[a];
      for (int j = a + 1; j <= b; ++j) v = fmaxf(v, S[j]);
    } else if (p.pool == 1) {
      float s = 0.0f;
      for (int j = a; j <= b; ++j) s += S[j];
      v = s / (float)p.pool_kernel;
    } else {
      v = S[i];
    }
    if (i < p.sink || i >= L - p.recent) v = INFINITY;
  }
  p.cand[(int64_t)seg * p.lv + p.kslot + x] = v;
}

// The kept slots (ascending) become the next running set: values into the
// next candidate row's first slots (-inf after the last kept), positions
// into pos_out.  `vt` is the step's selection plan (keff, out_off).
__global__ __launch_bounds__(NT) void stream_map_kernel(StreamParams p, SegTable vt) {
  const int sl = blockIdx.y;
  const int seg = vt.seg0 + sl;
  const int j = blockIdx.x * NT + threadIdx.x;
  if (j >= p.kslot) return;
  float *nxt = p.cand_next + (int64_t)seg * p.lv;
  if (j < vt.keff[sl]) {
    const int slot = p.sel[vt.out_off[sl] + j];
    const int pos = (slot < p.kslot) ? p.pos_in[(int64_t)seg * p.kslot + slot] : p.c0 + (slot - p.kslot);
    p.pos_out[(int64_t)seg * p.kslot + j] = pos;
    nxt[j] = p.cand[(int64_t)seg * p.lv + slot];
  } else {
    nxt[j] = -INFINITY;
  }
}

// After the last step: the running positions are the result.
__global__ __launch_bounds__(NT) void stream_final_kernel(StreamParams p, SegTable t, int32_t *idx) {
  const int sl = blockIdx.y;
  const int seg = t.seg0 + sl;
  const int j = blockIdx.x * NT + threadIdx.x;
  if (j < t.keff[sl]) idx[t.out_off[sl] + j] = p.pos_in[(int64_t)seg * p.kslot + j];
}

}  // namespace

hipError_t launch_stream_init(const StreamParams &p, const SegTable &t, hipStream_t s) {
  if (p.kslot <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_init_kernel, dim3((p.kslot + NT - 1) / NT, t.nseq * p.Hkv), dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

hipError_t launch_stream_pool(const StreamParams &p, const SegTable &t, hipStream_t s) {
  hipLaunchKernelGGL(stream_pool_kernel, dim3((p.stream + NT - 1) / NT, t.nseq * p.Hkv), dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

hipError_t launch_stream_map(const StreamParams &p, const SegTable &vt, hipStream_t s) {
  if (p.kslot <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_map_kernel, dim3((p.kslot + NT - 1) / NT, vt.nseq * p.Hkv), dim3(NT), 0, s, p, vt);
  return hipGetLastError();
}

hipError_t launch_stream_final(const StreamParams &p, const SegTable &t, int32_t *idx, hipStream_t s) {
  if (t.kmax <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_final_kernel, dim3((t.kmax + NT - 1) / NT, t.nseq * p.Hkv), dim3(NT), 0, s, p, t, idx);
  return hipGetLastError();
}

}  // namespace kvsel
