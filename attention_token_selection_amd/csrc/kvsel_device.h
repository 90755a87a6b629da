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

// tau, the rest-th largest of the m keys cand[0, m) in LDS (1 <= rest <= m
// <= 2 NTH), and take_eq, how many of the keys equal to tau are among the
// rest largest, into out[0] and out[1]: each key's count of larger and of
// equal keys, by comparison with all of them (every thread of a wave reads
// the same LDS words, which the LDS broadcasts); the key whose larger count
// is below rest and whose larger-or-equal count reaches it is tau (every
// such key is the same).  Each key's comparisons are split over S = NTH / m
// threads (at most 8), each taking a share of the keys in whole 16-byte
// reads, so that few keys still keep every wave busy; part (max(NTH, m)
// words of LDS) holds the shares' counts.  cand is padded with zeros to a
// multiple of 4 (its room must allow that); the padding is subtracted from
// the equal count of a zero key.  Every thread of the workgroup calls it.
template <int NTH>
__device__ void rank_select(uint32_t *cand, int m, int rest, uint32_t *part, int *out) {
  const int tid = threadIdx.x;
  const int m4 = (m + 3) & ~3;
  for (int i = m + tid; i < m4; i += NTH) cand[i] = 0u;
  __syncthreads();
  const int n4 = m4 >> 2;
  const int S = min(8, max(1, NTH / m));
  const int per = (n4 + S - 1) / S;  // 16-byte reads per share
  const uint4 *c4 = reinterpret_cast<const uint4 *>(cand);
  for (int t = tid; t < S * m; t += NTH) {
    const int sg = t / m, i = t - sg * m;
    const uint32_t ki = cand[i];
    uint32_t gt = 0u, eq = 0u;
    auto cmp = [&](const uint4 kj) {
      gt += (kj.x > ki) + (kj.y > ki) + (kj.z > ki) + (kj.w > ki);
      eq += (kj.x == ki) + (kj.y == ki) + (kj.z == ki) + (kj.w == ki);
    };
    const int q1 = min(n4, (sg + 1) * per);
    int q = sg * per;
    for (; q + 4 <= q1; q += 4) {  // four reads in flight
      const uint4 k0 = c4[q], k1 = c4[q + 1], k2 = c4[q + 2], k3 = c4[q + 3];
      cmp(k0);
      cmp(k1);
      cmp(k2);
      cmp(k3);
    }
    for (; q < q1; ++q) cmp(c4[q]);
    part[sg * m + i] = gt | (eq << 16);  // both at most m + 3 < 2^16
  }
  __syncthreads();
  for (int i = tid; i < m; i += NTH) {
    int gt = 0, eq = 0;
    for (int sg = 0; sg < S; ++sg) {
      const uint32_t w = part[sg * m + i];
      gt += (int)(w & 0xffffu);
      eq += (int)(w >> 16);
    }
    const uint32_t ki = cand[i];
    eq -= (ki == 0u) ? (m4 - m) : 0;  // the padding keys are 0
    if (gt < rest && gt + eq >= rest) {
      out[0] = (int)ki;
      out[1] = rest - gt;
    }
  }
  __syncthreads();
}

}  // namespace kvsel
