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
//
// The fused streaming form (pools up to 2 kPoolHalo + 1 wide) keeps the
// running set in a row of order keys instead: pass 2 with the pool writes
// each step's keys behind the running ones, and stream_select_kernel, one
// workgroup per segment with every key of the row in registers, picks the
// best keff in one launch per step (see there).
#include "kvsel_internal.h"
#include "kvsel_device.h"

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

// ---------------------------------------------------------------- fused running top-k
constexpr int ST = 1024;       // threads of stream_select_kernel
constexpr int SW = ST / 64;    // its waves
constexpr int kRankMax = 512;  // candidates of the threshold bin ranked directly

// Exclusive prefix sum over the workgroup; also returns the total.
__device__ inline uint32_t exscan_st(uint32_t v, uint32_t *tmp, uint32_t &total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wid] = x;
  __syncthreads();
  uint32_t before = 0u, tot = 0u;
#pragma unroll
  for (int i = 0; i < SW; ++i) {
    const uint32_t s = tmp[i];
    before += (i < wid) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// One step of the running top-k of one segment (TideKV §4.2, streaming
// form): the best keep = min(keff, keys seen) of the row's valid keys, ties
// to the lower slot (the lower position: running slots hold ascending
// positions, all before the step's).  Thread tid holds slots
// [IPT tid, IPT tid + IPT) in registers.  The threshold key tau is found as
// in the whole-prefix selection: the bin b1 of the keep-th largest key by
// the first digit (steps of 2^16 from the key of the mean score), then tau
// among the keys of bin b1, by direct ranking when at most kRankMax, else by
// three radix rounds (11 + 11 + 10 bits); then one ordered compaction.
template <int IPT>
__global__ __launch_bounds__(ST) void stream_select_kernel(StreamSelectParams p, SegTable t) {
  static_assert(IPT % 4 == 0 && IPT <= 16, "whole uint4 loads; at most 16 keys in registers");
  __shared__ uint32_t hist[kTabBins];
  __shared__ __attribute__((aligned(16))) uint32_t cand[kRankMax];
  __shared__ uint32_t tmp[SW];
  __shared__ int sh[5];
  const int sl = blockIdx.x;
  const int sb = sl / p.Hkv;
  const int seg = t.seg0 + sl;
  const int L = (int)(t.key_off[sb + 1] - t.key_off[sb]);
  const int keff = t.keff[sl];
  if (keff <= 0) return;  // the whole workgroup leaves together
  const int n_in = min(keff, min(L, p.c0));          // running keys
  const int m = max(0, min(p.stream, L - p.c0));     // this step's keys
  const int keep = min(keff, n_in + m);
  const int tid = threadIdx.x;
  const int i0 = tid * IPT;

  // ---- the thread's slots (past the row: a clamped re-read, invalid)
  const uint32_t *row = p.keys_in + (int64_t)seg * p.lv;
  uint32_t k[IPT];
#pragma unroll
  for (int j = 0; j < IPT; j += 4) {
    const uint4 u = *reinterpret_cast<const uint4 *>(row + min(i0 + j, p.lv - 4));
    k[j] = u.x;
    k[j + 1] = u.y;
    k[j + 2] = u.z;
    k[j + 3] = u.w;
  }
  // the running slots' positions (clamped; unused past the running
  // slots), loaded with the keys so that their latency overlaps the rest
  int32_t pv[IPT];
  if (p.kslot >= 4) {
    const int32_t *pin = p.pos_in + (int64_t)seg * p.kslot;
#pragma unroll
    for (int j = 0; j < IPT; j += 4) {
      const int4 u = *reinterpret_cast<const int4 *>(pin + min(i0 + j, p.kslot - 4));
      pv[j] = u.x;
      pv[j + 1] = u.y;
      pv[j + 2] = u.z;
      pv[j + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < IPT; ++j) pv[j] = 0;
  }
  uint32_t vm = 0u;  // bit j: slot i0 + j holds a key
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = i0 + j;
    vm |= (i < n_in || (i >= p.kslot && i < p.kslot + m)) ? (1u << j) : 0u;
  }

  // ---- tau and take_eq (keys equal to tau to keep, the first in slot
  // order); keeping every valid key: tau = 0, below every valid key
  uint32_t tau = 0u;
  int take_eq = 0;
  if (keep < n_in + m) {
    const uint32_t centre = order_key(p.wsum / (float)L);
    // monotone in the key: steps of 2^16 counted from the centre's step
    const int cstep = (int)(centre >> kTabDigitShift);
    auto digit = [&](uint32_t key) {
      return min(kTabBins - 1, max(0, (int)(key >> kTabDigitShift) - cstep + kTabBins / 2));
    };
    for (int i = tid; i < kTabBins; i += ST) hist[i] = 0u;
    if (tid == 0) sh[2] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if ((vm >> j) & 1u) atomicAdd(&hist[digit(k[j])], 1u);
    __syncthreads();
    // b1: thread tid owns bins 2 tid, 2 tid + 1
    const uint32_t h0 = hist[2 * tid], h1 = hist[2 * tid + 1];
    uint32_t tot;
    uint32_t below = exscan_st(h0 + h1, tmp, tot);  // keys in lower bins
    {
      const int ge0 = (int)(tot - below);  // keys in bins >= 2 tid
      const int ge1 = ge0 - (int)h0;       // ... >= 2 tid + 1
      const int ge2 = ge1 - (int)h1;       // ... >= 2 tid + 2
      if (ge0 >= keep && ge1 < keep) {
        sh[0] = 2 * tid;
        sh[1] = ge1;
      }
      if (ge1 >= keep && ge2 < keep) {
        sh[0] = 2 * tid + 1;
        sh[1] = ge2;
      }
    }
    __syncthreads();
    const int b1 = sh[0];
    int rest = keep - sh[1];  // keys of bin b1 to keep, >= 1
    // bin b1's keys as a key range (the edge bins take everything beyond;
    // a bin that holds a key has a step in [0, 2^16))
    const uint32_t b1step = (uint32_t)(b1 - kTabBins / 2 + cstep) << kTabDigitShift;
    const uint32_t klo = (b1 == 0) ? 0u : b1step;
    const uint32_t khi = (b1 == kTabBins - 1) ? 0xffffffffu : (b1step | ((1u << kTabDigitShift) - 1u));
    auto in_b1 = [&](uint32_t key) { return key >= klo && key <= khi; };
    // the candidates appended a wave at a time: one LDS atomic per wave and
    // slot with candidates (same-address atomics from many lanes serialize)
    const int lane = tid & 63;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const bool is_c = ((vm >> j) & 1u) && in_b1(k[j]);
      const uint64_t bal = __ballot(is_c);
      if (bal) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&sh[2], __popcll(bal));
        base = __shfl(base, 0);
        const int c = base + __popcll(bal & ((1ull << lane) - 1ull));
        if (is_c && c < kRankMax) cand[c] = k[j];
      }
    }
    __syncthreads();
    const int mc = sh[2];  // keys in bin b1
    if (mc <= kRankMax) {
      // by direct ranking, the comparisons spread over the workgroup
      rank_select<ST>(cand, mc, rest, hist, sh + 3);
      tau = (uint32_t)sh[3];
      take_eq = sh[4];
    } else {
      uint32_t pre = 0u;
      for (int hi = 32, lo = 21;; hi = lo, lo = (lo > 11) ? lo - 11 : 0) {
        for (int i = tid; i < kTabBins; i += ST) hist[i] = 0u;
        __syncthreads();
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
          if (((vm >> j) & 1u) && in_b1(k[j]) && (hi == 32 || (k[j] >> hi) == pre))
            atomicAdd(&hist[(k[j] >> lo) & dmask], 1u);
        }
        __syncthreads();
        const uint32_t g0 = hist[2 * tid], g1 = hist[2 * tid + 1];
        uint32_t gt2;
        const uint32_t ex = exscan_st(g0 + g1, tmp, gt2);
        int ab = (int)(gt2 - ex - g0 - g1);  // keys in bins above this thread's
        if (ab < rest && ab + (int)g1 >= rest) {
          sh[3] = 2 * tid + 1;
          sh[4] = ab;
        }
        ab += (int)g1;
        if (ab < rest && ab + (int)g0 >= rest) {
          sh[3] = 2 * tid;
          sh[4] = ab;
        }
        __syncthreads();
        rest -= sh[4];
        pre = (pre << (hi - lo)) | (uint32_t)sh[3];
        __syncthreads();
        if (lo == 0) break;
      }
      tau = pre;
      take_eq = rest;
    }
  }

  // ---- ordered compaction: slot order is position order
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const bool v = (vm >> j) & 1u;
    gt += (v && k[j] > tau) ? 1u : 0u;
    eq += (v && k[j] == tau) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t packed = exscan_st((gt << 16) | eq, tmp, tot);  // both counts stay below 2^16
  int eb = (int)(packed & 0xffffu);  // keys equal to tau in earlier threads' slots
  int slot = (int)(packed >> 16) + min(eb, take_eq);
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = i0 + j;
    const bool v = (vm >> j) & 1u;
    const bool is_eq = v && k[j] == tau;
    const bool kp = (v && k[j] > tau) || (is_eq && eb < take_eq);
    if (kp && slot < keep) {
      const int pos = (i < p.kslot) ? pv[j] : p.c0 + (i - p.kslot);
      if (p.last) {
        p.idx[t.out_off[sl] + slot] = pos;
      } else {
        p.keys_out[(int64_t)seg * p.lv + slot] = k[j];
        p.pos_out[(int64_t)seg * p.kslot + slot] = pos;
      }
    }
    slot += kp ? 1 : 0;
    eb += is_eq ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_stream_select(const StreamSelectParams &p, const SegTable &t, hipStream_t s) {
  if (p.lv < 4 || p.lv % 4 != 0 || p.kslot % 4 != 0 || p.lv > kStreamRowMax || p.kslot + p.stream > p.lv)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)(t.nseq * p.Hkv));
  const int ipt = (p.lv + ST - 1) / ST;
  if (ipt <= 4) hipLaunchKernelGGL(stream_select_kernel<4>, grid, dim3(ST), 0, s, p, t);
  else if (ipt <= 8) hipLaunchKernelGGL(stream_select_kernel<8>, grid, dim3(ST), 0, s, p, t);
  else hipLaunchKernelGGL(stream_select_kernel<16>, grid, dim3(ST), 0, s, p, t);
  return hipGetLastError();
}

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
