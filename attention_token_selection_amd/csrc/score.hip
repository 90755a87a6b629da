// Two-pass blockwise scoring of every prefix key against the observation rows
// (TideKV, "Delayed KV Eviction via Layer-Wise Chunked Prefill", §4.2).
//
// Work unit: one workgroup per (key block, KV head, sequence).  Inside it,
// waves are split into `nrg` row groups (4 row tiles = 64 observation rows
// each) times `ks` key splits (interleaved 16-key tiles).  Every wave keeps
// its rows' query fragments in registers for the whole block and streams its
// key tiles from HBM straight into MFMA operands:
//
//   D[16 rows x 16 keys] += Q[16 rows x 32 dims] * K^T[32 dims x 16 keys]
//   (v_mfma_f32_16x16x32_bf16, four k-steps cover d = 128).
//
// The contraction index may be permuted freely as long as Q and K agree, so
// lane group q = lane/16 of k-step j supplies the 16-byte chunk q + 4j of a
// 256-byte row: one load instruction then reads 64 contiguous bytes from each
// of 16 keys, and the four k-steps read every byte of the row once.
//
// Pass 1 keeps, per accumulator slot (row, key lane), a reference r and
// Z = sum 2^(x - r) of the base-2 logits x = s * scale * log2(e).  A slot's
// reference only moves when a new logit exceeds it by more than 2^16, checked
// once per tile for the whole wave, so the common path costs one FMA, one
// exp2 and one add per logit.  Slots merge with the log-sum-exp rule, first
// across lanes, then across key splits, then -- in the last workgroup of a
// (sequence, head) to arrive -- across key blocks, in a fixed order, giving
// per row bias = r + log2(Z) - log2(c_r).
//
// Pass 2 recomputes the logits and adds 2^(x - bias) over the wave's rows
// in-lane, across lane groups with two butterflies, and across row groups in
// LDS, in a fixed order (no floating-point atomics: results are
// bit-reproducible).
#include "kvsel_internal.h"

namespace kvsel {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr float kLazyThreshold = 16.0f;  // log2 units a logit may exceed its slot reference

__device__ inline bf16x8 load_frag(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(p));
}

__device__ inline bf16x8 zero_frag() { return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u)); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (r, z) <- merge of two partial log-sum-exp states in base 2.  Symmetric in
// its operands bit for bit, so butterfly partners agree exactly.
__device__ inline void lse_merge(float &r, float &z, float r2, float z2) {
  const float m = fmaxf(r, r2);
  if (m == -INFINITY) return;
  const float a = (r == -INFINITY) ? 0.0f : z * fast_exp2(r - m);
  const float b = (r2 == -INFINITY) ? 0.0f : z2 * fast_exp2(r2 - m);
  r = m;
  z = a + b;
}

// Arrival ticket of a (sequence, head) for the last-arriver merge.  A ticket
// is (kTicketTag << 32 | arrivals so far); the last arriver resets it to
// (kTicketTag << 32 | 0), so between calls every ticket reads "tag, 0" and an
// arrival is one fetch-add.  A ticket without the tag (a fresh workspace
// holding arbitrary bytes) is claimed once with a compare-and-swap; arrivals
// that raced onto the untagged value are discarded by that swap and redone.
constexpr uint32_t kTicketTag = 0x6b76736cu;

__device__ bool arrive_last(unsigned long long *ticket, uint32_t n) {
  const unsigned long long tag = (unsigned long long)kTicketTag << 32;
  unsigned long long old = __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  uint32_t count;
  if ((uint32_t)(old >> 32) == kTicketTag) {
    count = (uint32_t)old + 1u;
  } else {
    unsigned long long cur = old + 1ull;
    for (;;) {
      if ((uint32_t)(cur >> 32) == kTicketTag) {
        old = __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        count = (uint32_t)old + 1u;
        break;
      }
      if (__hip_atomic_compare_exchange_strong(ticket, &cur, tag | 1ull, __ATOMIC_ACQ_REL, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        count = 1u;
        break;
      }
    }
  }
  if (count == n) {
    __hip_atomic_store(ticket, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  return false;
}

// Key fragments of this lane's key.  The key index is clamped into the
// sequence so every load is in bounds and branch-free; keys past the end are
// masked in the epilogue.
__device__ inline void load_key_tile(bf16x8 (&kf)[4], const uint16_t *kbase, int64_t key0, int L, int Hkv,
                                     int key) {
  const int kk = min(key, L - 1);
  const uint16_t *src = kbase + (key0 + kk) * Hkv * (int64_t)kHeadDim;
#pragma unroll
  for (int j = 0; j < 4; ++j) kf[j] = load_frag(src + 32 * j);
}

// RT: row tiles held per wave (the launch spreads the row tiles evenly over
// the row groups; tiles past the last row hold zero queries).
template <int PASS, int RT>
__global__ __launch_bounds__(512) void score_kernel(ScoreParams p, SegTable t) {
  extern __shared__ float lds[];
  __shared__ int s_last;

  const int blk = blockIdx.x;
  const int h = blockIdx.y;
  const int sb = blockIdx.z;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  const int kb0 = blk * p.key_block;
  if (kb0 >= L) return;  // the whole workgroup leaves together
  const int kb1 = min(L, kb0 + p.key_block);
  const int seg = t.seg0 + sb * p.Hkv + h;
  const int b = t.seq0 + sb;

  // wave-uniform indices (scalar registers, scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rg = wave % p.nrg;
  const int ks = wave / p.nrg;
  const int lq = lane >> 4;  // lane group: rows 4*lq.. of a D tile, chunk group of A/B
  const int lc = lane & 15;  // key column of a D tile, row of an A tile

  // Query fragments of this wave's row tiles (rows = window row major,
  // query head of the group minor).
  bf16x8 qf[RT][4];
#pragma unroll
  for (int tt = 0; tt < RT; ++tt) {
    const int row = (rg * RT + tt) * kTile + lc;
    if (row < p.R) {
      const int r = row / p.G;
      const int gi = row - r * p.G;
      const uint16_t *src =
          p.Q + ((int64_t)(b * p.wp + r) * p.Hq + h * p.G + gi) * (int64_t)kHeadDim + lq * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) qf[tt][j] = load_frag(src + 32 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) qf[tt][j] = zero_frag();
    }
  }

  // Last visible key of each accumulator slot's row (causal limit, and the
  // end of the sequence for every row).
  int lim[RT][4];
  float bias[RT][4];
  float ref[RT][4], zs[RT][4];
#pragma unroll
  for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = (rg * RT + tt) * kTile + 4 * lq + e;
      const int r = row / p.G;
      const int pos = (r < p.w) ? (L - p.w + r) : L;
      lim[tt][e] = p.causal ? min(pos, L - 1) : (L - 1);
      ref[tt][e] = -INFINITY;
      zs[tt][e] = 0.0f;
      bias[tt][e] = (PASS == 2) ? p.bias[(int64_t)seg * p.Rpad + row] : 0.0f;
    }
  }

  const int ntile = (kb1 - kb0 + kTile - 1) / kTile;
  const int mask_from = p.causal ? (L - p.w) : L;
  const float cl2 = p.cl2;
  const int step = p.ks;
  const uint16_t *kbase = p.K + (int64_t)h * kHeadDim + lq * 8;

  auto tile = [&](const bf16x8(&kf)[4], int ti) {
    const int i0 = kb0 + ti * kTile;
    f32x4 acc[RT];
#pragma unroll
    for (int tt = 0; tt < RT; ++tt) acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int tt = 0; tt < RT; ++tt)
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[tt][j], kf[j], acc[tt], 0, 0, 0);
    }

    const bool need_mask = (i0 + kTile) > mask_from;
    const int key = i0 + lc;

    if constexpr (PASS == 1) {
      float tv[RT][4];
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = fmaf(acc[tt][e], cl2, -ref[tt][e]);
          if (need_mask && key > lim[tt][e]) v = -INFINITY;
          tv[tt][e] = v;
          mx = fmaxf(mx, v);
        }
      }
      if (__ballot(mx > kLazyThreshold) != 0ull) {
        // Rare: some logit outgrew its slot's reference; move references up.
#pragma unroll
        for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (need_mask && key > lim[tt][e]) continue;
            const float x = acc[tt][e] * cl2;
            if (x > ref[tt][e]) {
              zs[tt][e] = (ref[tt][e] == -INFINITY) ? 0.0f : zs[tt][e] * fast_exp2(ref[tt][e] - x);
              ref[tt][e] = x;
            }
            tv[tt][e] = x - ref[tt][e];
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) zs[tt][e] += fast_exp2(tv[tt][e]);
      }
    } else {
      float sum = 0.0f;
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = fast_exp2(fmaf(acc[tt][e], cl2, -bias[tt][e]));
          if (need_mask && key > lim[tt][e]) v = 0.0f;
          sum += v;
        }
      }
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      if (lq == 0) lds[rg * p.key_block + (i0 - kb0) + lc] = sum;
    }
  };

  // Two key tiles in flight per wave (ping-pong), every load unconditional.
  bf16x8 ka[4], kb[4];
  load_key_tile(ka, kbase, key0, L, p.Hkv, kb0 + ks * kTile + lc);
  for (int ti = ks; ti < ntile; ti += 2 * step) {
    load_key_tile(kb, kbase, key0, L, p.Hkv, kb0 + (ti + step) * kTile + lc);
    tile(ka, ti);
    load_key_tile(ka, kbase, key0, L, p.Hkv, kb0 + (ti + 2 * step) * kTile + lc);
    if (ti + step < ntile) tile(kb, ti + step);
  }

  if constexpr (PASS == 2) {
    __syncthreads();
    const int n = kb1 - kb0;
    float *out = p.scores + (int64_t)p.Hkv * key0 + (int64_t)h * L + kb0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      float v = 0.0f;
      for (int g = 0; g < p.nrg; ++g) v += lds[g * p.key_block + i];
      out[i] = v;
    }
    return;
  } else {
    // Merge the 16 key lanes that share each row (butterfly, symmetric).
#pragma unroll
    for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float r2 = __shfl_xor(ref[tt][e], off);
          const float z2 = __shfl_xor(zs[tt][e], off);
          lse_merge(ref[tt][e], zs[tt][e], r2, z2);
        }
      }
    }
    float2 *st = reinterpret_cast<float2 *>(lds);  // [ks][Rpad]
    if (lc == 0) {
#pragma unroll
      for (int tt = 0; tt < RT; ++tt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = (rg * RT + tt) * kTile + 4 * lq + e;
          st[ks * p.Rpad + row] = make_float2(ref[tt][e], zs[tt][e]);
        }
      }
    }
    __syncthreads();
    const int nblk_seg = (L + p.key_block - 1) / p.key_block;
    float2 *part = p.partials + ((int64_t)seg * p.nblk1_max + blk) * p.Rpad;
    for (int row = threadIdx.x; row < p.Rpad; row += blockDim.x) {
      float r = -INFINITY, z = 0.0f;
      for (int k2 = 0; k2 < p.ks; ++k2) {
        const float2 v = st[k2 * p.Rpad + row];
        lse_merge(r, z, v.x, v.y);
      }
      part[row] = make_float2(r, z);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = arrive_last(&p.tickets[seg - t.seg0], (uint32_t)nblk_seg) ? 1 : 0;
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float2 *all = p.partials + (int64_t)seg * p.nblk1_max * p.Rpad;
    for (int row = threadIdx.x; row < p.Rpad; row += blockDim.x) {
      float r = -INFINITY, z = 0.0f;
      for (int bb = 0; bb < nblk_seg; ++bb) {
        const float2 v = all[(int64_t)bb * p.Rpad + row];
        lse_merge(r, z, v.x, v.y);
      }
      const int wr = row / p.G;
      float c = 1.0f;
      if (p.has_decode) c = (wr < p.w) ? (1.0f - p.alpha) : p.alpha;
      float out = INFINITY;
      if (row < p.R && c > 0.0f && z > 0.0f) out = r + log2f(z) - log2f(c);
      p.bias[(int64_t)seg * p.Rpad + row] = out;
    }
  }
}

template <int PASS>
hipError_t launch_pass(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s, size_t lds) {
  const dim3 grid(nblk, p.Hkv, t.nseq);
  const dim3 block(64 * p.nrg * p.ks);
  switch (p.rt) {
    case 1: hipLaunchKernelGGL((score_kernel<PASS, 1>), grid, block, lds, s, p, t); break;
    case 2: hipLaunchKernelGGL((score_kernel<PASS, 2>), grid, block, lds, s, p, t); break;
    case 3: hipLaunchKernelGGL((score_kernel<PASS, 3>), grid, block, lds, s, p, t); break;
    default: hipLaunchKernelGGL((score_kernel<PASS, 4>), grid, block, lds, s, p, t); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_pass1(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  return launch_pass<1>(p, t, nblk, s, (size_t)p.ks * p.Rpad * sizeof(float2));
}

hipError_t launch_score_pass2(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  return launch_pass<2>(p, t, nblk, s, (size_t)p.nrg * p.key_block * sizeof(float));
}

}  // namespace kvsel
