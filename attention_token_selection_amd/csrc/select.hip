// Pool + top-k of one (sequence, KV head) segment per workgroup.
//
// The 1-D pool (odd width, stride 1; avg = zero-padded sum / width, max over
// in-range positions) is applied while the segment is read once; the pooled
// values are written out and their order keys feed an LDS histogram.
//
// Selection is a three-digit radix select (11 + 11 + 10 bits) on order keys
// of the fp32 values (monotone: larger value, larger key; -0 ranks as +0).
// It finds the k-th largest key tau and how many of the keys equal to tau
// are needed.  Compaction then walks the segment in index order: each thread
// owns a contiguous run, a block-wide exclusive scan of its (greater, equal)
// counts gives its first output slot, and an element is kept if its key is
// greater than tau, or equal to tau and among the first needed equal ones.
// This keeps the lower position among equal scores and emits positions in
// ascending order (TideKV §5 keeps original positions; the DeferKV guide,
// Phase 3, sorts the kept indices) -- no sort is needed.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int NT = kSelectThreads;
constexpr int NWAVE = NT / 64;

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float pooled_at(const float *S, int L, int i, int pool, int r, float width) {
  if (pool == 0 || r == 0) return S[i];
  if (pool == 1) {
    float s = 0.0f;
    for (int j = i - r; j <= i + r; ++j)
      if (j >= 0 && j < L) s += S[j];
    return s / width;
  }
  const int lo = max(0, i - r), hi = min(L - 1, i + r);
  float m = S[lo];
  for (int j = lo + 1; j <= hi; ++j) m = fmaxf(m, S[j]);
  return m;
}

// Exclusive prefix sum over the workgroup; also returns the total.
__device__ int block_exscan(int v, int *tmp, int &total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  int before = 0, tot = 0;
  for (int i = 0; i < NWAVE; ++i) {
    const int s = tmp[i];
    before += (i < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// Bin holding the need-th largest element of the histogram, and the number
// of elements in higher bins.
__device__ void find_bin(const uint32_t *hist, int nbins, int need, int *tmp, int *s_bin, int *s_above,
                         int &bin, int &above) {
  const int per = nbins / NT;
  const int first = threadIdx.x * per;
  int c = 0;
  for (int j = 0; j < per; ++j) c += (int)hist[first + j];
  int total;
  const int pre = block_exscan(c, tmp, total);
  int ab = total - pre - c;
  for (int j = per - 1; j >= 0; --j) {
    const int hb = (int)hist[first + j];
    if (ab < need && ab + hb >= need) {
      *s_bin = first + j;
      *s_above = ab;
    }
    ab += hb;
  }
  __syncthreads();
  bin = *s_bin;
  above = *s_above;
  __syncthreads();
}

__global__ __launch_bounds__(NT) void pool_topk_kernel(SelectParams p, SegTable t) {
  __shared__ uint32_t hist[2048];
  __shared__ int tmp[NWAVE];
  __shared__ int s_bin, s_above;

  const int h = blockIdx.x;
  const int sb = blockIdx.y;
  const int segl = sb * p.Hkv + h;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  const int64_t base = (int64_t)p.Hkv * key0 + (int64_t)h * L;
  const float *S = p.scores + base;
  float *P = p.pooled + base;
  int32_t *out = p.idx + t.out_off[segl];
  const int keff = t.keff[segl];
  const int r = (p.pool == 0) ? 0 : (p.pool_kernel - 1) / 2;
  const float width = (float)p.pool_kernel;
  const int tid = threadIdx.x;

  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < L; i += NT) {
    const float v = pooled_at(S, L, i, p.pool, r, width);
    P[i] = v;
    atomicAdd(&hist[order_key(v) >> 21], 1u);
  }
  __syncthreads();
  if (keff <= 0) return;
  if (keff >= L) {
    for (int i = tid; i < L; i += NT) out[i] = i;
    return;
  }

  int need = keff, bin1, bin2, bin3, above;
  find_bin(hist, 2048, need, tmp, &s_bin, &s_above, bin1, above);
  need -= above;

  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < L; i += NT) {
    const uint32_t k = order_key(P[i]);
    if ((int)(k >> 21) == bin1) atomicAdd(&hist[(k >> 10) & 2047u], 1u);
  }
  __syncthreads();
  find_bin(hist, 2048, need, tmp, &s_bin, &s_above, bin2, above);
  need -= above;

  const uint32_t pre22 = ((uint32_t)bin1 << 11) | (uint32_t)bin2;
  for (int i = tid; i < 1024; i += NT) hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < L; i += NT) {
    const uint32_t k = order_key(P[i]);
    if ((k >> 10) == pre22) atomicAdd(&hist[k & 1023u], 1u);
  }
  __syncthreads();
  find_bin(hist, 1024, need, tmp, &s_bin, &s_above, bin3, above);
  need -= above;

  const uint32_t tau = (pre22 << 10) | (uint32_t)bin3;
  const int take_eq = need;  // >= 1 by construction

  const int chunk = (L + NT - 1) / NT;
  const int lo = min(L, tid * chunk), hi = min(L, lo + chunk);
  int gt = 0, eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t k = order_key(P[i]);
    gt += (k > tau);
    eq += (k == tau);
  }
  int tot;
  const int gt_before = block_exscan(gt, tmp, tot);
  const int eq_before = block_exscan(eq, tmp, tot);
  int pos = gt_before + min(eq_before, take_eq);
  int eq_seen = eq_before;
  for (int i = lo; i < hi; ++i) {
    const uint32_t k = order_key(P[i]);
    if (k > tau) {
      if (pos < keff) out[pos] = i;
      ++pos;
    } else if (k == tau) {
      if (eq_seen < take_eq) {
        if (pos < keff) out[pos] = i;
        ++pos;
      }
      ++eq_seen;
    }
  }
}

}  // namespace

hipError_t launch_pool_topk(const SelectParams &p, const SegTable &t, hipStream_t s) {
  const dim3 grid(p.Hkv, t.nseq);
  hipLaunchKernelGGL(pool_topk_kernel, grid, dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel
