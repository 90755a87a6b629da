// Pool + top-k of one (sequence, KV head) segment per workgroup.
//
// The segment is processed in pieces of 8192 positions (8 consecutive
// positions per thread).  For each piece the scores plus a halo of
// (width-1)/2 on each side are staged into LDS with coalesced loads, and the
// 1-D pool (odd width, stride 1; avg = zero-padded sum / width, max over
// in-range positions) is evaluated from LDS.  Pooled values are written out
// and, for segments up to 8 pieces long, kept in registers for the selection
// passes; longer segments re-read them from memory.
//
// Selection is a three-digit radix select (11 + 11 + 10 bits) on order keys
// of the fp32 values (monotone: larger value, larger key; -0 ranks as +0).
// It finds the k-th largest key tau and how many of the keys equal to tau
// are needed.  Compaction walks the pieces in order; inside a piece each
// thread owns 8 consecutive positions, and a block-wide exclusive scan of the
// packed (greater, equal) counts gives each thread its first output slot.  A
// position is kept if its key is greater than tau, or equal to tau and among
// the first needed equal ones -- so the lower position wins among equal
// scores and positions come out ascending (TideKV §5 keeps original
// positions; the DeferKV guide, Phase 3, sorts the kept indices), without a
// sort.
#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int NT = kSelectThreads;
constexpr int NWAVE = NT / 64;
constexpr int PER = 8;              // positions per thread per piece
constexpr int PIECE = NT * PER;     // positions per piece
constexpr int HALO = (kMaxPoolKernel - 1) / 2;

__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
#pragma unroll
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

// NP > 0: at most NP pieces, pooled values kept in registers.
// NP == 0: any length, pooled values re-read from memory on each pass.
template <int NP>
__global__ __launch_bounds__(NT) void pool_topk_kernel(SelectParams p, SegTable t) {
  __shared__ float stage[PIECE + 2 * HALO];
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
  const int npieces = (L + PIECE - 1) / PIECE;

  constexpr int NR = NP > 0 ? NP : 1;
  float reg[NR][PER];

  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;

  // ---- pool every piece, write it out, histogram of the top 11 key bits
  auto pool_piece = [&](int pc, float (&v)[PER]) {
    const int plo = pc * PIECE;
    const int span = PIECE + 2 * r;
    __syncthreads();  // previous piece's stage reads are done
    for (int j = tid; j < span; j += NT) {
      const int gi = plo - r + j;
      stage[j] = (gi >= 0 && gi < L) ? S[gi] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int li = tid * PER + e;  // position within the piece
      const int i = plo + li;
      float x = 0.0f;
      if (i < L) {
        if (r == 0) {
          x = stage[li];
        } else if (p.pool == 1) {
          float s = 0.0f;
          for (int j = -r; j <= r; ++j) s += stage[li + r + j];  // outside positions are staged as 0
          x = s / width;
        } else {
          const int lo = max(-r, -i), hi = min(r, L - 1 - i);
          x = stage[li + r + lo];
          for (int j = lo + 1; j <= hi; ++j) x = fmaxf(x, stage[li + r + j]);
        }
        P[i] = x;
        atomicAdd(&hist[order_key(x) >> 21], 1u);
      }
      v[e] = x;
    }
  };

  if constexpr (NP > 0) {
#pragma unroll
    for (int pc = 0; pc < NP; ++pc)
      if (pc < npieces) pool_piece(pc, reg[pc]);
  } else {
    for (int pc = 0; pc < npieces; ++pc) pool_piece(pc, reg[0]);
  }
  __syncthreads();
  if (keff <= 0) return;
  if (keff >= L) {
    for (int i = tid; i < L; i += NT) out[i] = i;
    return;
  }

  // Visit every valid (position, pooled value) of this thread in piece order.
  auto for_each = [&](auto &&fn) {
    if constexpr (NP > 0) {
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) {
        if (pc < npieces) {
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            const int i = pc * PIECE + tid * PER + e;
            if (i < L) fn(reg[pc][e]);
          }
        }
      }
    } else {
      for (int pc = 0; pc < npieces; ++pc) {
        float v[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int i = pc * PIECE + tid * PER + e;
          v[e] = (i < L) ? P[i] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < PER; ++e)
          if (pc * PIECE + tid * PER + e < L) fn(v[e]);
      }
    }
  };

  int need = keff, bin1, bin2, bin3, above;
  find_bin(hist, 2048, need, tmp, &s_bin, &s_above, bin1, above);
  need -= above;

  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
  __syncthreads();
  for_each([&](float x) {
    const uint32_t k = order_key(x);
    if ((int)(k >> 21) == bin1) atomicAdd(&hist[(k >> 10) & 2047u], 1u);
  });
  __syncthreads();
  find_bin(hist, 2048, need, tmp, &s_bin, &s_above, bin2, above);
  need -= above;

  const uint32_t pre22 = ((uint32_t)bin1 << 11) | (uint32_t)bin2;
  for (int i = tid; i < 1024; i += NT) hist[i] = 0u;
  __syncthreads();
  for_each([&](float x) {
    const uint32_t k = order_key(x);
    if ((k >> 10) == pre22) atomicAdd(&hist[k & 1023u], 1u);
  });
  __syncthreads();
  find_bin(hist, 1024, need, tmp, &s_bin, &s_above, bin3, above);
  need -= above;

  const uint32_t tau = (pre22 << 10) | (uint32_t)bin3;
  const int take_eq = need;  // >= 1 by construction

  // ---- ordered compaction, one piece at a time
  int g_before = 0, e_before = 0;  // counts in earlier pieces (workgroup-uniform)
  auto compact_piece = [&](int pc, const float (&v)[PER]) {
    uint32_t key[PER];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = pc * PIECE + tid * PER + e;
      key[e] = (i < L) ? order_key(v[e]) : 0u;
      gt += (i < L) && key[e] > tau;
      eq += (i < L) && key[e] == tau;
    }
    int total;
    const int packed = block_exscan((gt << 16) | eq, tmp, total);
    int gb = g_before + (packed >> 16);
    int eb = e_before + (packed & 0xffff);
    int pos = gb + min(eb, take_eq);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = pc * PIECE + tid * PER + e;
      if (i >= L) continue;
      if (key[e] > tau) {
        if (pos < keff) out[pos] = i;
        ++pos;
      } else if (key[e] == tau) {
        if (eb < take_eq) {
          if (pos < keff) out[pos] = i;
          ++pos;
        }
        ++eb;
      }
    }
    g_before += total >> 16;
    e_before += total & 0xffff;
  };
  if constexpr (NP > 0) {
#pragma unroll
    for (int pc = 0; pc < NP; ++pc)
      if (pc < npieces) compact_piece(pc, reg[pc]);
  } else {
    for (int pc = 0; pc < npieces; ++pc) {
      float v[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int i = pc * PIECE + tid * PER + e;
        v[e] = (i < L) ? P[i] : 0.0f;
      }
      compact_piece(pc, v);
    }
  }
}

}  // namespace

hipError_t launch_pool_topk(const SelectParams &p, const SegTable &t, hipStream_t s) {
  int64_t lmax = 0;
  for (int i = 0; i < t.nseq; ++i) lmax = std::max<int64_t>(lmax, t.key_off[i + 1] - t.key_off[i]);
  const int64_t pieces = (lmax + PIECE - 1) / PIECE;
  const dim3 grid(p.Hkv, t.nseq);
  if (pieces <= 1)
    hipLaunchKernelGGL(pool_topk_kernel<1>, grid, dim3(NT), 0, s, p, t);
  else if (pieces <= 2)
    hipLaunchKernelGGL(pool_topk_kernel<2>, grid, dim3(NT), 0, s, p, t);
  else if (pieces <= 4)
    hipLaunchKernelGGL(pool_topk_kernel<4>, grid, dim3(NT), 0, s, p, t);
  else if (pieces <= 8)
    hipLaunchKernelGGL(pool_topk_kernel<8>, grid, dim3(NT), 0, s, p, t);
  else
    hipLaunchKernelGGL(pool_topk_kernel<0>, grid, dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel
