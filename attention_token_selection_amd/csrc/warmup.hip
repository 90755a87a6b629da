// Importance-guided warm-up ("KVDrive: A Holistic Multi-Tier KV Cache
// Management System for Long-Context LLM Inference", §7.1): one importance
// value per prefix position, the aggregated observation-window scores summed
// over the KV heads of every layer, and a three-tier placement from its
// ranking (fast tier, middle tier, backing store).
//
// profile_kernel: per sequence, out[i] = sum over heads h of S[h][i] (heads
// in order 0, 1, ..., so the sum is reproducible), plus the previous value
// when accumulating over layers.  One thread per position, all of its heads'
// loads in flight at once; the loads of a head are coalesced.
//
// tier_fill_kernel / tier_mark_kernel: the labels start at 2 (backing store
// only); the positions of a selection (from the pool and top-k kernels, run
// on the profile as one segment per sequence) are then overwritten with
// their tier, the middle tier's selection first and the fast tier's last.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int NT = 256;
constexpr int HBATCH = 8;  // heads loaded before they are summed

__global__ __launch_bounds__(NT) void profile_kernel(ProfileParams p, SegTable t) {
  const int sb = blockIdx.y;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  const int i = blockIdx.x * NT + threadIdx.x;
  if (i >= L) return;
  const float *S = p.scores + (int64_t)p.Hkv * key0 + i;
  float acc = 0.0f;
  for (int h0 = 0; h0 < p.Hkv; h0 += HBATCH) {
    float v[HBATCH];
#pragma unroll
    for (int u = 0; u < HBATCH; ++u) v[u] = (h0 + u < p.Hkv) ? S[(int64_t)(h0 + u) * L] : 0.0f;
#pragma unroll
    for (int u = 0; u < HBATCH; ++u) acc += v[u];  // heads in order; the padding adds +0
  }
  float *out = p.profile + key0 + i;
  *out = p.accumulate ? *out + acc : acc;
}

__global__ __launch_bounds__(NT) void tier_fill_kernel(int8_t *tier, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (i < n) tier[i] = 2;
}

// Writes `label` at the positions of each sequence's selection: segment sb
// of the selection holds keff[sb] positions (relative to the sequence start)
// from out_off[sb].
__global__ __launch_bounds__(NT) void tier_mark_kernel(const int32_t *idx, int8_t *tier, int8_t label, SegTable t) {
  const int sb = blockIdx.y;
  const int j = blockIdx.x * NT + threadIdx.x;
  if (j >= t.keff[sb]) return;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  const int pos = idx[t.out_off[sb] + j];
  if ((unsigned)pos < (unsigned)L) tier[key0 + pos] = label;
}

}  // namespace

hipError_t launch_profile(const ProfileParams &p, const SegTable &t, int64_t lmax, hipStream_t s) {
  if (lmax <= 0 || t.nseq <= 0) return hipSuccess;
  const dim3 grid((unsigned)((lmax + NT - 1) / NT), t.nseq);
  hipLaunchKernelGGL(profile_kernel, grid, dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

hipError_t launch_tier_fill(int8_t *tier, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(tier_fill_kernel, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, s, tier, n);
  return hipGetLastError();
}

hipError_t launch_tier_mark(const int32_t *idx, int8_t *tier, int label, const SegTable &t, hipStream_t s) {
  if (t.kmax <= 0 || t.nseq <= 0) return hipSuccess;
  const dim3 grid((unsigned)((t.kmax + NT - 1) / NT), t.nseq);
  hipLaunchKernelGGL(tier_mark_kernel, grid, dim3(NT), 0, s, idx, tier, (int8_t)label, t);
  return hipGetLastError();
}

}  // namespace kvsel
