// Pool + top-k (+ optionally the K/V compaction) of every (sequence, KV
// head) segment, in two launches whose workgroups each own one chunk of
// 2048 positions of one segment, so that every per-position step runs
// spread over the chip even when a launch holds only a few segments.
//
// 1. pool_bucket_kernel.  Pools the chunk (odd width, stride 1; avg =
//    zero-padded window sum / width, max over the in-range positions;
//    positions outside the sequence read as the pool's neutral value, 0 for
//    avg and -inf for max, so windows need no bounds logic) and writes it.
//    Then a counting sort of the chunk by the first radix digit of each
//    pooled value's order key (its top 13 bits): the exclusive prefix of the
//    chunk's digit histogram is written out (tab_fine, plus every 32nd entry
//    in tab_coarse) together with the chunk's keys grouped by digit
//    (bucket).  No global atomics; nothing needs clearing beforehand.
//
// 2. select_chunk_kernel.  Every workgroup of a segment first finds, from
//    the tables of all the segment's chunks, the digit b1 whose bin holds
//    the k-th largest key (a 256-way search over tab_coarse, then over 32
//    entries of tab_fine).  It loads the keys of bin b1 from every chunk's
//    bucket (usually a few hundred candidates) and resolves the remaining 19
//    bits with radix rounds over those candidates alone.  This gives tau,
//    the k-th largest key, and take_eq, how many keys equal to tau are kept:
//    the lowest-positioned ones.  Per-chunk counts of kept keys then give
//    each chunk's first output slot, and the workgroup writes the kept
//    positions of its own chunk in ascending order (a scan of packed
//    (greater, equal) counts), so positions come out sorted and the lower
//    position wins among equal scores (TideKV §5 keeps original positions;
//    the DeferKV guide, Phase 3, sorts the kept indices).  When K_out is
//    given it also copies the kept K and V rows to the compact layout
//    (TideKV §4.1 and §5); then two workgroups share each chunk, each
//    copying half of its rows, so the copy is spread over twice as many
//    compute units.
//
// Order keys: the fp32 bits mapped so that a larger value has a larger
// unsigned key (-0 ranks as +0); reserved positions (DeferKV guide, Phase 3:
// attention sinks and the recent window) take the largest key of all.
#include "kvsel_internal.h"
#include "kvsel_device.h"

namespace kvsel {
namespace {

constexpr int NT = 256;                  // threads of both kernels
constexpr int NWAVE = NT / 64;
constexpr int CH = kSelectChunk;         // positions per chunk (workgroup)
constexpr int PER = CH / NT;             // positions per thread
constexpr int NBIN = kSelectBins;        // first-digit bins
constexpr int DSHIFT = 19;               // first digit = key >> DSHIFT
constexpr int CSTEP = 32;                // tab_coarse keeps every CSTEP-th prefix entry
constexpr int NCOARSE = NBIN / CSTEP;    // = NT: one coarse entry per thread
constexpr int WIN = CSTEP + 1;           // staged prefix entries per chunk in the second search level
constexpr int MAXC = 4096;               // candidates held in LDS (more: re-read from memory)
constexpr int MAXCH = kMaxChunks;
constexpr int HALO = (kMaxPoolKernel - 1) / 2;
constexpr int HOFF = 128;                // stage index of a chunk's first position (>= HALO, multiple of 4)
constexpr int FASTR = 4;                 // pools of radius <= FASTR run from a register window
static_assert(PER == 8, "two 16-byte runs per thread");
static_assert(NBIN == 1 << (32 - DSHIFT), "first digit width");
static_assert(NCOARSE == NT, "one coarse entry per thread");
static_assert(HOFF >= HALO && HOFF % 4 == 0, "stage layout");
static_assert(MAXCH <= 2 * NT, "chunk scans hold two chunks per thread");

// N consecutive values of X from position `first` on (first may be
// negative), `fill` outside [0, L); 16-byte loads where the run is in range
// and aligned.
template <int N>
__device__ inline void load_run(const float *X, int L, int first, bool vec, float fill, float (&v)[N]) {
  if (vec && first >= 0 && first + N <= L) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const float4 a = *reinterpret_cast<const float4 *>(X + first + 4 * q);
      v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = (first + e >= 0 && first + e < L) ? X[first + e] : fill;
  }
}

template <int N>
__device__ inline void store_run(float *X, int L, int first, bool vec, const float (&v)[N]) {
  if (vec && first + N <= L) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q)
      *reinterpret_cast<float4 *>(X + first + 4 * q) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e)
      if (first + e < L) X[first + e] = v[e];
  }
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

// Number of threads of the workgroup for which `pred` holds.
__device__ int block_count(bool pred, int *tmp) {
  const int n = __popcll(__ballot(pred));
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = n;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) tot += tmp[i];
  __syncthreads();
  return tot;
}

// Sum of v over the workgroup (every thread gets it).
__device__ uint64_t block_sum64(uint64_t v, uint64_t *tmp64) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) tmp64[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) tot += tmp64[i];
  __syncthreads();
  return tot;
}

// Exclusive prefix sum of a 64-bit value over the workgroup (two 32-bit
// counts packed in one scan as one, while neither sum reaches 2^32); also
// returns the total.
__device__ uint64_t block_exscan64(uint64_t v, uint64_t *tmp64, uint64_t &total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint64_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp64[wid] = x;
  __syncthreads();
  uint64_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NWAVE; ++i) {
    const uint64_t s = tmp64[i];
    before += (i < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

struct Segment {
  const float *S;
  float *P;
  int32_t *out;
  int64_t key0;   // first key row of the sequence
  int64_t out0;   // first output row of the segment
  int seg;        // global segment index
  int h;
  int L, keff, r;
  bool is_max, vec_in, vec_out;
  float fill, width;
};

__device__ inline Segment segment_of(const SelectParams &p, const SegTable &t, int h, int sb) {
  Segment g;
  const int segl = sb * p.Hkv + h;
  g.key0 = t.key_off[sb];
  g.seg = t.seg0 + segl;
  g.h = h;
  g.L = (int)(t.key_off[sb + 1] - g.key0);
  const int64_t base = (int64_t)p.Hkv * g.key0 + (int64_t)h * g.L;
  g.S = p.scores + base;
  g.P = p.pooled + base;
  g.out0 = t.out_off[segl];
  g.out = p.idx + g.out0;
  g.keff = t.keff[segl];
  g.r = (p.pool == 0) ? 0 : (p.pool_kernel - 1) / 2;
  g.is_max = p.pool == 2;
  // Positions outside the sequence: 0 for the zero-padded average, -inf
  // (never the maximum: a window always holds its own in-range centre) for max.
  g.fill = g.is_max ? -INFINITY : 0.0f;
  g.width = (float)p.pool_kernel;
  g.vec_in = (reinterpret_cast<uintptr_t>(g.S) & 15u) == 0;
  g.vec_out = (reinterpret_cast<uintptr_t>(g.P) & 15u) == 0;
  return g;
}

__device__ inline int chunk_len(int L, int c) { return min(CH, L - c * CH); }

// ---------------------------------------------------------------- 1. pool + counting sort by first digit
__global__ __launch_bounds__(NT) void pool_bucket_kernel(SelectParams p, SegTable t) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[NBIN];  // counts, then exclusive prefix
  // Dynamic: HOFF + CH + HOFF floats for pools wider than 2 FASTR + 1,
  // nothing otherwise (the launch sizes it).
  extern __shared__ __attribute__((aligned(16))) float stage[];
  __shared__ int tmp[NWAVE];

  const Segment g = segment_of(p, t, blockIdx.y, blockIdx.z);
  const int c = blockIdx.x;
  const int p0 = c * CH;
  if (p0 >= g.L) return;  // the whole workgroup leaves together
  const int tid = threadIdx.x;
  const int first = p0 + tid * PER;

  uint4 *h4 = reinterpret_cast<uint4 *>(hist);
  for (int i = tid; i < NBIN / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);

  float v[PER];
  if (g.r == 0) {
    load_run<PER>(g.S, g.L, first, g.vec_in, g.fill, v);
  } else if (g.r <= FASTR) {
    float wv[PER + 2 * FASTR];
    load_run<PER + 2 * FASTR>(g.S, g.L, first - FASTR, g.vec_in, g.fill, wv);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (g.is_max) {
        float m = wv[FASTR + e];
#pragma unroll
        for (int j = -FASTR; j <= FASTR; ++j)
          if (j != 0 && j >= -g.r && j <= g.r) m = fmaxf(m, wv[FASTR + e + j]);
        v[e] = m;
      } else {
        float sum = 0.0f;
#pragma unroll
        for (int j = -FASTR; j <= FASTR; ++j)
          if (j >= -g.r && j <= g.r) sum += wv[FASTR + e + j];
        v[e] = sum / g.width;
      }
    }
  } else {
    const int span = CH + 2 * g.r;
    for (int j = tid; j < span; j += NT) {
      const int pos = p0 - g.r + j;
      stage[HOFF - g.r + j] = (pos >= 0 && pos < g.L) ? g.S[pos] : g.fill;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const float *cc = stage + HOFF + tid * PER + e;
      if (g.is_max) {
        float m = cc[0];
        for (int j = -g.r; j <= g.r; ++j) m = fmaxf(m, cc[j]);
        v[e] = m;
      } else {
        float sum = 0.0f;
        for (int j = -g.r; j <= g.r; ++j) sum += cc[j];
        v[e] = sum / g.width;
      }
    }
  }
  store_run<PER>(g.P, g.L, first, g.vec_out, v);

  // Histogram; the value an atomic returns is the position's rank in its bin.
  __syncthreads();  // the histogram is cleared
  uint32_t bin[PER], rank[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    bin[e] = select_key(v[e], first + e, g.L, p.sink, p.recent) >> DSHIFT;
    rank[e] = (first + e < g.L) ? atomicAdd(&hist[bin[e]], 1u) : 0u;
  }
  __syncthreads();

  // Exclusive prefix over the bins: thread tid owns bins [32 tid, 32 tid + 32).
  uint32_t cnt[CSTEP];
#pragma unroll
  for (int q = 0; q < CSTEP / 4; ++q) {
    const uint4 a = h4[tid * (CSTEP / 4) + q];
    cnt[4 * q] = a.x; cnt[4 * q + 1] = a.y; cnt[4 * q + 2] = a.z; cnt[4 * q + 3] = a.w;
  }
  int own = 0;
#pragma unroll
  for (int j = 0; j < CSTEP; ++j) own += (int)cnt[j];
  int total;
  uint32_t run = (uint32_t)block_exscan(own, tmp, total);  // its barriers also end the reads above
  uint32_t pre[CSTEP];
#pragma unroll
  for (int j = 0; j < CSTEP; ++j) {
    pre[j] = run;
    run += cnt[j];
  }
#pragma unroll
  for (int q = 0; q < CSTEP / 4; ++q)
    h4[tid * (CSTEP / 4) + q] = make_uint4(pre[4 * q], pre[4 * q + 1], pre[4 * q + 2], pre[4 * q + 3]);
  // Prefixes are at most CH = 2048: 16 bits hold them.
  const int64_t tab = (int64_t)g.seg * p.nchunk_max + c;
  uint4 *tf = reinterpret_cast<uint4 *>(p.tab_fine + tab * NBIN + tid * CSTEP);
#pragma unroll
  for (int q = 0; q < CSTEP / 8; ++q)
    tf[q] = make_uint4(pre[8 * q] | (pre[8 * q + 1] << 16), pre[8 * q + 2] | (pre[8 * q + 3] << 16),
                       pre[8 * q + 4] | (pre[8 * q + 5] << 16), pre[8 * q + 6] | (pre[8 * q + 7] << 16));
  p.tab_coarse[tab * NCOARSE + tid] = (uint16_t)pre[0];
  __syncthreads();

  uint32_t *bk = p.bucket + tab * CH;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (first + e < g.L) bk[hist[bin[e]] + rank[e]] = select_key(v[e], first + e, g.L, p.sink, p.recent);
}

// ---------------------------------------------------------------- 2. select + compaction per chunk
template <bool GATHER>
__global__ __launch_bounds__(NT) void select_chunk_kernel(SelectParams p, SegTable t) {
  __shared__ uint32_t candk[MAXC];       // keys of bin b1
  __shared__ uint16_t candc[MAXC];       // their chunks
  __shared__ uint32_t hist[2048];
  // Per-chunk arrays, in dynamic LDS sized for the launch's longest
  // sequence (nch_cap chunks; select_lds_bytes): a launch of short
  // sequences leaves room for several workgroups per compute unit.
  extern __shared__ __attribute__((aligned(16))) int dyn[];
  const int nch_cap = (int)gridDim.x / (GATHER ? 2 : 1);
  int *ch_lo = dyn;                        // per chunk: start of bin b1 in its bucket
  int *ch_cb = ch_lo + nch_cap;            // per chunk: first candidate index (nch_cap + 1)
  int *ch_above = ch_cb + nch_cap + 1;     // per chunk: keys in bins above b1
  int *ch_gt = ch_above + nch_cap;         // per chunk: candidates above tau
  int *ch_eq = ch_gt + nch_cap;            // per chunk: candidates equal to tau
  uint16_t (*win)[WIN] = reinterpret_cast<uint16_t (*)[WIN]>(ch_eq + nch_cap);  // per chunk: prefix entries 32 t0 .. 32 t0 + 32
  __shared__ int ge32[CSTEP];
  __shared__ uint16_t kept[CH];          // kept chunk-local positions, in output order
  __shared__ int tmp[NWAVE];
  __shared__ int sh[4];

  const Segment g = segment_of(p, t, blockIdx.y, blockIdx.z);
  // With the gather, two workgroups share a chunk: both select (the same
  // result), the first writes the indices, and each copies half the rows.
  const int c = GATHER ? (blockIdx.x >> 1) : blockIdx.x;
  const int half = GATHER ? (blockIdx.x & 1) : 0;
  const int p0 = c * CH;
  if (p0 >= g.L) return;  // the whole workgroup leaves together
  if (g.keff <= 0) return;
  const int tid = threadIdx.x;
  const int nch = (g.L + CH - 1) / CH;
  const int n_me = chunk_len(g.L, c);
  const int first = p0 + tid * PER;

  int base = 0;   // first output slot of this chunk
  int nkept = 0;  // kept positions of this chunk
  if (g.keff >= g.L) {
    base = p0;
    nkept = n_me;
    for (int i = tid; i < n_me; i += NT) {
      if (half == 0) g.out[p0 + i] = p0 + i;
      kept[i] = (uint16_t)i;
    }
  } else {
    // This chunk's pooled values, for the compaction at the end (issued now,
    // used last).
    float v[PER];
    load_run<PER>(g.P, g.L, first, g.vec_out, 0.0f, v);

    const int64_t tab0 = (int64_t)g.seg * p.nchunk_max;
    const uint16_t *TC = p.tab_coarse + tab0 * NCOARSE;
    const uint16_t *TF = p.tab_fine + tab0 * NBIN;
    const uint32_t *BK = p.bucket + tab0 * CH;

    // ---- b1: the largest digit b with ge(b) >= keff, where ge(b) counts
    // the segment's keys whose digit is >= b (over chunks: length - prefix).
    int ge1 = 0;  // ge(32 tid)
    for (int c0 = 0; c0 < nch; c0 += 16) {
      uint32_t e[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) e[u] = (c0 + u < nch) ? TC[(int64_t)(c0 + u) * NCOARSE + tid] : 0u;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c0 + u < nch) ge1 += chunk_len(g.L, c0 + u) - (int)e[u];
    }
    if (tid == 0) sh[0] = 0;
    const int t0 = block_count(ge1 >= g.keff, tmp) - 1;  // >= 0 because ge(0) = L > keff
    if (tid == t0 + 1) sh[0] = ge1;                       // ge(32 (t0 + 1)); 0 past the last bin
    // Stage prefix entries 32 t0 .. 32 t0 + 32 of every chunk (entry NBIN,
    // past the last bin, is the chunk's length).
    for (int f0 = 0; f0 < nch * WIN; f0 += 4 * NT) {
      uint32_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = f0 + u * NT + tid;
        const int cc = f / WIN, jj = f - (f / WIN) * WIN, b = CSTEP * t0 + jj;
        e[u] = (f < nch * WIN) ? ((b < NBIN) ? TF[(int64_t)cc * NBIN + b] : (uint32_t)chunk_len(g.L, cc)) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int f = f0 + u * NT + tid;
        if (f < nch * WIN) win[f / WIN][f - (f / WIN) * WIN] = (uint16_t)e[u];
      }
    }
    __syncthreads();
    const int j = tid >> 3, q = tid & 7;  // bin 32 t0 + j; chunks q, q + 8, ...
    int ge2 = 0;
    for (int cc = q; cc < nch; cc += 8) ge2 += chunk_len(g.L, cc) - (int)win[cc][j];
    ge2 += __shfl_xor(ge2, 1);
    ge2 += __shfl_xor(ge2, 2);
    ge2 += __shfl_xor(ge2, 4);
    if (q == 0) ge32[j] = ge2;
    const int j1 = block_count(q == 0 && ge2 >= g.keff, tmp) - 1;  // >= 0
    const int b1 = CSTEP * t0 + j1;
    const int ge_next = (j1 + 1 < CSTEP) ? ge32[j1 + 1] : sh[0];
    const int need = g.keff - ge_next;  // keys of bin b1 to keep, >= 1
    const int m = ge32[j1] - ge_next;   // keys in bin b1, >= need

    // ---- per-chunk extent of bin b1, and candidate offsets
    for (int cc = tid; cc < nch; cc += NT) {
      const int lo = win[cc][j1], hi = win[cc][j1 + 1];
      ch_lo[cc] = lo;
      ch_above[cc] = chunk_len(g.L, cc) - hi;
      ch_gt[cc] = 0;
      ch_eq[cc] = 0;
      ch_cb[cc] = hi - lo;
    }
    __syncthreads();
    {
      const int a = (2 * tid < nch) ? ch_cb[2 * tid] : 0;
      const int b = (2 * tid + 1 < nch) ? ch_cb[2 * tid + 1] : 0;
      int tot;
      const int ex = block_exscan(a + b, tmp, tot);
      if (2 * tid < nch) ch_cb[2 * tid] = ex;
      if (2 * tid + 1 < nch) ch_cb[2 * tid + 1] = ex + a;
      if (tid == 0) ch_cb[nch] = tot;  // = m
    }
    __syncthreads();

    // Candidate i lives in chunk cc (the largest cc with ch_cb[cc] <= i).
    auto cand_chunk = [&](int i) {
      int lo = 0, hi = nch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ch_cb[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      return lo;
    };
    auto cand_addr = [&](int i, int cc) { return (int64_t)cc * CH + ch_lo[cc] + (i - ch_cb[cc]); };
    const bool in_lds = m <= MAXC;
    if (in_lds) {
      for (int i0 = 0; i0 < m; i0 += 4 * NT) {
        uint32_t k[4];
        int cc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * NT + tid;
          cc[u] = (i < m) ? cand_chunk(i) : 0;
          k[u] = (i < m) ? BK[cand_addr(i, cc[u])] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * NT + tid;
          if (i < m) {
            candk[i] = k[u];
            candc[i] = (uint16_t)cc[u];
          }
        }
      }
      __syncthreads();
    }
    auto visit = [&](auto &&fn) {
      for (int i = tid; i < m; i += NT) {
        if (in_lds) {
          fn(candk[i], (int)candc[i]);
        } else {
          const int cc = cand_chunk(i);
          fn(BK[cand_addr(i, cc)], cc);
        }
      }
    };

    // ---- radix rounds below b1: bits [8, 19), then [0, 8)
    int rest = need;
    uint32_t pre = (uint32_t)b1;
    for (int hi = DSHIFT, lo = DSHIFT - 11;; hi = lo, lo = 0) {
      for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
      __syncthreads();
      const uint32_t dmask = (1u << (hi - lo)) - 1u;
      visit([&](uint32_t k, int) {
        if ((k >> hi) == pre) atomicAdd(&hist[(k >> lo) & dmask], 1u);
      });
      __syncthreads();
      // The bin holding the rest-th largest: thread tid owns bins [8 tid, 8 tid + 8).
      uint32_t hc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) hc[u] = hist[8 * tid + u];
      int own = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) own += (int)hc[u];
      int tot;
      const int ex = block_exscan(own, tmp, tot);
      int ab = tot - ex - own;  // keys in bins above this thread's
#pragma unroll
      for (int u = 7; u >= 0; --u) {
        if (ab < rest && ab + (int)hc[u] >= rest) {
          sh[1] = 8 * tid + u;
          sh[2] = ab;
        }
        ab += (int)hc[u];
      }
      __syncthreads();
      rest -= sh[2];
      pre = (pre << (hi - lo)) | (uint32_t)sh[1];
      __syncthreads();
      if (lo == 0) break;
    }
    const uint32_t tau = pre;
    const int take_eq = rest;  // keys equal to tau to keep (the lowest-positioned), >= 1

    // ---- per-chunk kept counts, and this chunk's first output slot
    visit([&](uint32_t k, int cc) {
      if (k > tau) atomicAdd(&ch_gt[cc], 1);
      else if (k == tau) atomicAdd(&ch_eq[cc], 1);
    });
    __syncthreads();
    int take_me;  // keys equal to tau that this chunk keeps
    {
      const int e0 = (2 * tid < nch) ? ch_eq[2 * tid] : 0;
      const int e1 = (2 * tid + 1 < nch) ? ch_eq[2 * tid + 1] : 0;
      int tot;
      const int ex = block_exscan(e0 + e1, tmp, tot);  // equal keys in earlier chunks
      const int k0 = min(e0, max(0, take_eq - ex));
      const int k1 = min(e1, max(0, take_eq - ex - e0));
      const int s0 = (2 * tid < nch) ? ch_above[2 * tid] + ch_gt[2 * tid] + k0 : 0;
      const int s1 = (2 * tid + 1 < nch) ? ch_above[2 * tid + 1] + ch_gt[2 * tid + 1] + k1 : 0;
      const int sx = block_exscan(s0 + s1, tmp, tot);
      if (2 * tid == c) {
        sh[1] = sx;
        sh[3] = k0;
      }
      if (2 * tid + 1 == c) {
        sh[1] = sx + s0;
        sh[3] = k1;
      }
      __syncthreads();
      base = sh[1];
      take_me = sh[3];
    }

    // ---- ordered compaction of this chunk
    uint32_t k[PER];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool valid = first + e < g.L;
      k[e] = select_key(v[e], first + e, g.L, p.sink, p.recent);
      gt += (valid && k[e] > tau) ? 1 : 0;
      eq += (valid && k[e] == tau) ? 1 : 0;
    }
    int tot;
    const int packed = block_exscan((gt << 16) | eq, tmp, tot);
    int eb = packed & 0xffff;  // keys equal to tau before this thread's, in this chunk
    int slot = (packed >> 16) + min(eb, take_me);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool valid = first + e < g.L;
      const bool is_eq = valid && k[e] == tau;
      const bool keep = (valid && k[e] > tau) || (is_eq && eb < take_me);
      if (keep && base + slot < g.keff) {  // always true; keeps every store inside the segment
        if (half == 0) g.out[base + slot] = first + e;
        kept[slot] = (uint16_t)(tid * PER + e);
      }
      slot += keep ? 1 : 0;
      eb += is_eq ? 1 : 0;
    }
    nkept = min((tot >> 16) + min(tot & 0xffff, take_me), g.keff - base);
  }

  if constexpr (GATHER) {
    // Copy this workgroup's half of the kept rows (rows 2 r + half): 16
    // lanes move one 256-byte row of K and of V, four rows per lane group in
    // flight.  Rows past the end repeat the last row (the same bytes to the
    // same place), so every load and store is unconditional.
    __syncthreads();
    const int part = tid & 15;
    const int nmine = (nkept - half + 1) / 2;  // rows 2 r + half, r < nmine
    constexpr int GR = NT / 16;                // lane groups
    auto row_of = [&](int r) { return 2 * min(r, nmine - 1) + half; };
    auto src = [&](int r) { return ((g.key0 + p0 + kept[row_of(r)]) * p.Hkv + g.h) * 16 + part; };
    auto dst = [&](int r) { return (g.out0 + base + row_of(r)) * 16 + part; };
    for (int r0 = tid >> 4; r0 < nmine; r0 += 4 * GR) {
      const int64_t s0 = src(r0), s1 = src(r0 + GR), s2 = src(r0 + 2 * GR), s3 = src(r0 + 3 * GR);
      const uint4 k0 = p.K[s0], k1 = p.K[s1], k2 = p.K[s2], k3 = p.K[s3];
      const uint4 v0 = p.V[s0], v1 = p.V[s1], v2 = p.V[s2], v3 = p.V[s3];
      p.K_out[dst(r0)] = k0;
      p.V_out[dst(r0)] = v0;
      p.K_out[dst(r0 + GR)] = k1;
      p.V_out[dst(r0 + GR)] = v1;
      p.K_out[dst(r0 + 2 * GR)] = k2;
      p.V_out[dst(r0 + 2 * GR)] = v2;
      p.K_out[dst(r0 + 3 * GR)] = k3;
      p.V_out[dst(r0 + 3 * GR)] = v3;
    }
  }
}


// ---------------------------------------------------------------- selection from pass 2's tables
// Pass 2 with tables leaves, per block of RBP = 256 positions, the
// exclusive prefix of the block's first-digit histogram (a monotone
// function of the order key; tab_fine, u16 [NB2]) and the block's keys
// grouped by digit (bucket, u32 [RBP]), plus each segment's whole digit
// histogram (seg_hist).  One workgroup per chunk of CH positions (CPB
// blocks) takes the steps of select_chunk_kernel: b1 straight from the
// segment's histogram; the keys of bin b1 from every block's bucket; their
// whole 32-bit keys in three radix rounds (11 + 11 + 10 bits) over those
// candidates; per-block kept counts; the chunk's ordered compaction and,
// with K_out, the copy.  The digit function itself is never needed here.
constexpr int RBP = kTabBlock;
constexpr int CPB = CH / RBP;            // blocks per chunk
constexpr int NB2 = kTabBins;
constexpr int BPT = 16;                  // blocks per thread in the per-block scans
constexpr int kRankCands = 512;          // at most this many candidates: tau by direct ranking
constexpr int MAXB = BPT * NT;           // blocks per segment: 4096, so up to 2^20 positions
static_assert(CPB == 8 && BPT == 2 * CPB, "a chunk's blocks are one half of a thread's share");
static_assert(NB2 == 8 * NT, "eight bins per thread");
static_assert((int64_t)MAXB * RBP >= (int64_t)MAXCH * CH, "every supported sequence fits the per-block scans");

template <bool GATHER>
__global__ __launch_bounds__(NT) void select_block_kernel(SelectParams p, SegTable t) {
  __shared__ __attribute__((aligned(16))) uint32_t candk[MAXC];  // keys of bin b1
  __shared__ uint16_t candb[MAXC];       // their blocks
  __shared__ uint32_t hist[2048];
  // Per-block arrays in dynamic LDS, sized for the launch's longest sequence.
  extern __shared__ __attribute__((aligned(16))) int dyn[];
  const int nb_cap = (int)gridDim.x / (GATHER ? 2 : 1) * CPB;
  int *b_lo = dyn;                        // per block: start of bin b1 in its bucket
  int *b_cb = b_lo + nb_cap;              // per block: first candidate index (nb_cap + 1)
  int *b_above = b_cb + nb_cap + 1;       // per block: keys in bins above b1
  int *b_gt = b_above + nb_cap;           // per block: candidates above tau
  int *b_eq = b_gt + nb_cap;              // per block: candidates equal to tau
  __shared__ uint16_t kept[CH];           // kept chunk-local positions, in output order
  __shared__ int tmp[NWAVE];
  __shared__ int sh[4];

  const Segment g = segment_of(p, t, blockIdx.y, blockIdx.z);
  const int c = GATHER ? (blockIdx.x >> 1) : blockIdx.x;
  const int half = GATHER ? (blockIdx.x & 1) : 0;
  const int p0 = c * CH;
  if (p0 >= g.L) return;  // the whole workgroup leaves together
  if (g.keff <= 0) return;
  const int tid = threadIdx.x;
  const int nb = (g.L + RBP - 1) / RBP;
  const int n_me = chunk_len(g.L, c);
  const int first = p0 + tid * PER;

  int base = 0;   // first output slot of this chunk
  int nkept = 0;  // kept positions of this chunk
  if (g.keff >= g.L) {
    base = p0;
    nkept = n_me;
    for (int i = tid; i < n_me; i += NT) {
      if (half == 0) g.out[p0 + i] = p0 + i;
      kept[i] = (uint16_t)i;
    }
  } else {
    float v[PER];
    load_run<PER>(g.P, g.L, first, g.vec_out, 0.0f, v);

    const int64_t tab0 = (int64_t)g.seg * p.nblk_max;
    const uint16_t *TF = p.tab_fine + tab0 * NB2;
    const uint32_t *BK = p.bucket + tab0 * RBP;

    // ---- b1: the digit b with ge(b) >= keff > ge(b + 1), where ge(b)
    // counts the segment's keys whose digit is >= b.
    if (tid == 0) {
      sh[0] = 0;
      sh[1] = 0;
    }
    {
      uint32_t cnt[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
      for (int cp = 0; cp < kTabHistCopies; ++cp) {  // the histogram's copies add up to it
        const uint4 *SH = reinterpret_cast<const uint4 *>(p.seg_hist + ((int64_t)g.seg * kTabHistCopies + cp) * NB2);
        const uint4 a0 = SH[2 * tid], a1 = SH[2 * tid + 1];
        cnt[0] += a0.x; cnt[1] += a0.y; cnt[2] += a0.z; cnt[3] += a0.w;
        cnt[4] += a1.x; cnt[5] += a1.y; cnt[6] += a1.z; cnt[7] += a1.w;
      }
      int own = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) own += (int)cnt[u];
      int tot;
      int below = block_exscan(own, tmp, tot);  // keys in lower bins; tot = L
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ge = tot - below;
        const int gn = ge - (int)cnt[u];
        if (ge >= g.keff && gn < g.keff) {
          sh[0] = 8 * tid + u;
          sh[1] = gn;
        }
        below += (int)cnt[u];
      }
      __syncthreads();
    }
    const int b1 = sh[0];
    const int need = g.keff - sh[1];  // keys of bin b1 to keep, >= 1

    // ---- per-block extent of bin b1, and candidate offsets
    if (nb <= NT) {
      // one block per thread: the prefixes of both counts (candidates; keys
      // above bin b1) in one packed scan, straight from the loads
      const int j = tid;
      uint32_t cbj = 0u, abj = 0u;
      if (j < nb) {
        const int len = min(RBP, g.L - j * RBP);
        const int lo = TF[(int64_t)j * NB2 + b1];
        const int hi = (b1 + 1 < NB2) ? (int)TF[(int64_t)j * NB2 + b1 + 1] : len;
        b_lo[j] = lo;
        b_above[j] = len - hi;
        b_gt[j] = 0;
        b_eq[j] = 0;
        cbj = (uint32_t)(hi - lo);
        abj = (uint32_t)(len - hi);
      }
      __shared__ uint64_t tmpx[NWAVE];
      uint64_t tot;
      const uint64_t ex = block_exscan64(((uint64_t)abj << 32) | cbj, tmpx, tot);  // each sum < 2^32
      if (j < nb) b_cb[j] = (int)(uint32_t)ex;
      if (j == 0) b_cb[nb] = (int)(uint32_t)tot;
      if (j == CPB * c) sh[2] = (int)(ex >> 32);  // the chunk's first block (< nb)
      __syncthreads();
    } else {
      for (int j = tid; j < nb; j += NT) {
        const int len = min(RBP, g.L - j * RBP);
        const int lo = TF[(int64_t)j * NB2 + b1];
        const int hi = (b1 + 1 < NB2) ? (int)TF[(int64_t)j * NB2 + b1 + 1] : len;
        b_lo[j] = lo;
        b_above[j] = len - hi;
        b_cb[j] = hi - lo;
        b_gt[j] = 0;
        b_eq[j] = 0;
      }
      __syncthreads();
      {
        // exclusive prefix over the blocks of the candidate counts: thread tid
        // owns blocks [BPT tid, BPT tid + BPT); and the keys above bin b1 in
        // the blocks before this chunk's (CPB c onwards: one half of thread
        // c / 2's share)
        int a[BPT], s = 0, sa = 0, ah = 0;
        const int h0 = (c & 1) * CPB;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
          const int j = BPT * tid + u;
          a[u] = (j < nb) ? b_cb[j] : 0;
          s += a[u];
          const int ab = (j < nb) ? b_above[j] : 0;
          sa += ab;
          ah += (u < h0) ? ab : 0;
        }
        int tot;
        int ex = block_exscan(s, tmp, tot);
        int tota;
        const int exa = block_exscan(sa, tmp, tota);
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
          const int j = BPT * tid + u;
          if (j < nb) b_cb[j] = ex;
          ex += a[u];
        }
        if (tid == 0) b_cb[nb] = tot;
        if (tid == (c >> 1)) sh[2] = exa + ah;
      }
      __syncthreads();
    }
    const int above_before = sh[2];  // keys above bin b1 in blocks [0, CPB c)
    const int m = b_cb[nb];  // keys in bin b1, >= need

    // Candidate i lives in block j (the largest j with b_cb[j] <= i).
    auto cand_block = [&](int i) {
      int lo = 0, hi = nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (b_cb[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      return lo;
    };
    auto cand_addr = [&](int i, int j) { return (int64_t)j * RBP + b_lo[j] + (i - b_cb[j]); };
    const bool in_lds = m <= MAXC;
    if (in_lds) {
      for (int i0 = 0; i0 < m; i0 += 4 * NT) {
        uint32_t k[4];
        int jb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * NT + tid;
          jb[u] = (i < m) ? cand_block(i) : 0;
          k[u] = (i < m) ? BK[cand_addr(i, jb[u])] : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * NT + tid;
          if (i < m) {
            candk[i] = k[u];
            candb[i] = (uint16_t)jb[u];
          }
        }
      }
      __syncthreads();
    }
    auto visit = [&](auto &&fn) {
      for (int i = tid; i < m; i += NT) {
        if (in_lds) {
          fn(candk[i], (int)candb[i]);
        } else {
          const int j = cand_block(i);
          fn(BK[cand_addr(i, j)], j);
        }
      }
    };

    // ---- tau, the need-th largest candidate key, and take_eq, how many of
    // the keys equal to it are kept (the lowest-positioned ones).  Few
    // candidates (held in LDS): by direct ranking (rank_select).  Otherwise
    // radix rounds over the candidates' keys: bits [21, 32), [10, 21), [0, 10).
    uint32_t tau;
    int take_eq;
    if (in_lds && m <= kRankCands) {
      rank_select<NT>(candk, m, need, hist, sh + 2);
      tau = (uint32_t)sh[2];
      take_eq = sh[3];
    } else {
      // ---- radix rounds over the candidates' keys: bits [21, 32), [10, 21), [0, 10)
      int rest = need;
      uint32_t pre = 0u;
      for (int hi = 32, lo = 21;; hi = lo, lo = (lo > 11) ? lo - 11 : 0) {
        for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
        __syncthreads();
        const uint32_t dmask = (1u << (hi - lo)) - 1u;
        visit([&](uint32_t k, int) {
          if (hi == 32 || (k >> hi) == pre) atomicAdd(&hist[(k >> lo) & dmask], 1u);
        });
        __syncthreads();
        // The bin holding the rest-th largest: thread tid owns bins [8 tid, 8 tid + 8).
        uint32_t hc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) hc[u] = hist[8 * tid + u];
        int own = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) own += (int)hc[u];
        int tot;
        const int ex = block_exscan(own, tmp, tot);
        int ab = tot - ex - own;  // keys in bins above this thread's
#pragma unroll
        for (int u = 7; u >= 0; --u) {
          if (ab < rest && ab + (int)hc[u] >= rest) {
            sh[2] = 8 * tid + u;
            sh[3] = ab;
          }
          ab += (int)hc[u];
        }
        __syncthreads();
        rest -= sh[3];
        pre = (pre << (hi - lo)) | (uint32_t)sh[2];
        __syncthreads();
        if (lo == 0) break;
      }
      tau = pre;
      take_eq = rest;
    }

    // ---- this chunk's first output slot and its share of the keys equal
    // to tau.  Candidates in LDS: the kept keys before the chunk are those
    // above bin b1 there, the candidates there above tau and the first
    // take_eq equal to it (lower blocks first); one sum over the
    // candidates.  Otherwise per-block counts and two scans over the blocks.
    int take_me;  // keys equal to tau that this chunk keeps
    if (in_lds) {
      const int cb0 = CPB * c, cb1 = cb0 + CPB;
      uint64_t gtb = 0, eqb = 0, eqi = 0;  // candidates > tau before the chunk, == tau before it, == tau in it
      for (int i = tid; i < m; i += NT) {
        const uint32_t k = candk[i];
        const int j = candb[i];
        gtb += (j < cb0 && k > tau) ? 1u : 0u;
        eqb += (j < cb0 && k == tau) ? 1u : 0u;
        eqi += (j >= cb0 && j < cb1 && k == tau) ? 1u : 0u;
      }
      __shared__ uint64_t tmp64[NWAVE];
      const uint64_t packed = block_sum64(gtb | (eqb << 21) | (eqi << 42), tmp64);  // each count <= MAXC < 2^21
      const int gt_before = (int)(packed & 0x1fffff);
      const int eq_before = (int)((packed >> 21) & 0x1fffff);
      const int eq_in = (int)(packed >> 42);
      base = above_before + gt_before + min(eq_before, take_eq);
      take_me = max(0, min(eq_in, take_eq - eq_before));
    } else {
      visit([&](uint32_t k, int j) {
        if (k > tau) atomicAdd(&b_gt[j], 1);
        else if (k == tau) atomicAdd(&b_eq[j], 1);
      });
      __syncthreads();
      {
        int e[BPT], es = 0;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
          const int j = BPT * tid + u;
          e[u] = (j < nb) ? b_eq[j] : 0;
          es += e[u];
        }
        int tot;
        int eb = block_exscan(es, tmp, tot);  // equal keys in earlier blocks
        int tk[BPT], sk[BPT], ss = 0;
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
          const int j = BPT * tid + u;
          tk[u] = min(e[u], max(0, take_eq - eb));
          eb += e[u];
          sk[u] = (j < nb) ? b_above[j] + b_gt[j] + tk[u] : 0;
          ss += sk[u];
        }
        int sb = block_exscan(ss, tmp, tot);
        // The chunk's blocks CPB c .. CPB c + CPB - 1 are one half of thread
        // c / 2's share: its first half for even c, its second for odd c.
        if (tid == (c >> 1)) {
          const int h0 = (c & 1) * CPB;
          int tm = 0;
#pragma unroll
          for (int u = 0; u < BPT; ++u) {
            sb += (u < h0) ? sk[u] : 0;
            tm += (u >= h0 && u < h0 + CPB) ? tk[u] : 0;
          }
          sh[2] = sb;
          sh[3] = tm;
        }
        __syncthreads();
      }
      base = sh[2];
      take_me = sh[3];
    }

    // ---- ordered compaction of this chunk
    uint32_t k[PER];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool valid = first + e < g.L;
      k[e] = select_key(v[e], first + e, g.L, p.sink, p.recent);
      gt += (valid && k[e] > tau) ? 1 : 0;
      eq += (valid && k[e] == tau) ? 1 : 0;
    }
    int tot;
    const int packed = block_exscan((gt << 16) | eq, tmp, tot);
    int eb = packed & 0xffff;  // keys equal to tau before this thread's, in this chunk
    int slot = (packed >> 16) + min(eb, take_me);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool valid = first + e < g.L;
      const bool is_eq = valid && k[e] == tau;
      const bool keep = (valid && k[e] > tau) || (is_eq && eb < take_me);
      if (keep && base + slot < g.keff) {  // always true; keeps every store inside the segment
        if (half == 0) g.out[base + slot] = first + e;
        kept[slot] = (uint16_t)(tid * PER + e);
      }
      slot += keep ? 1 : 0;
      eb += is_eq ? 1 : 0;
    }
    nkept = min((tot >> 16) + min(tot & 0xffff, take_me), g.keff - base);
  }

  if constexpr (GATHER) {
    // Copy this workgroup's half of the kept rows (rows 2 r + half), as in
    // select_chunk_kernel.
    __syncthreads();
    const int part = tid & 15;
    const int nmine = (nkept - half + 1) / 2;
    constexpr int GR = NT / 16;
    auto row_of = [&](int r) { return 2 * min(r, nmine - 1) + half; };
    auto src = [&](int r) { return ((g.key0 + p0 + kept[row_of(r)]) * p.Hkv + g.h) * 16 + part; };
    auto dst = [&](int r) { return (g.out0 + base + row_of(r)) * 16 + part; };
    for (int r0 = tid >> 4; r0 < nmine; r0 += 4 * GR) {
      const int64_t s0 = src(r0), s1 = src(r0 + GR), s2 = src(r0 + 2 * GR), s3 = src(r0 + 3 * GR);
      const uint4 k0 = p.K[s0], k1 = p.K[s1], k2 = p.K[s2], k3 = p.K[s3];
      const uint4 v0 = p.V[s0], v1 = p.V[s1], v2 = p.V[s2], v3 = p.V[s3];
      p.K_out[dst(r0)] = k0;
      p.V_out[dst(r0)] = v0;
      p.K_out[dst(r0 + GR)] = k1;
      p.V_out[dst(r0 + GR)] = v1;
      p.K_out[dst(r0 + 2 * GR)] = k2;
      p.V_out[dst(r0 + 2 * GR)] = v2;
      p.K_out[dst(r0 + 3 * GR)] = k3;
      p.V_out[dst(r0 + 3 * GR)] = v3;
    }
  }
}

}  // namespace

// Dynamic LDS of select_chunk_kernel for a launch whose longest sequence
// has `nch` chunks: five int arrays (one with an extra entry) and the
// prefix-entry windows.
static size_t select_lds_bytes(int nch) {
  return (size_t)(5 * nch + 1) * sizeof(int) + (size_t)nch * WIN * sizeof(uint16_t);
}

hipError_t launch_pool_topk(const SelectParams &p, const SegTable &t, hipStream_t s) {
  int64_t lmax = 0;
  for (int i = 0; i < t.nseq; ++i) lmax = std::max<int64_t>(lmax, t.key_off[i + 1] - t.key_off[i]);
  const int nch = (int)((lmax + CH - 1) / CH);
  if (nch < 1 || nch > MAXCH) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nch, p.Hkv, t.nseq);
  const int r = (p.pool == 0) ? 0 : (p.pool_kernel - 1) / 2;
  const size_t stage = (r > FASTR) ? (size_t)(HOFF + CH + HOFF) * sizeof(float) : 0;
  hipLaunchKernelGGL(pool_bucket_kernel, grid, dim3(NT), stage, s, p, t);
  if (p.K_out)
    hipLaunchKernelGGL(select_chunk_kernel<true>, dim3(2 * grid.x, grid.y, grid.z), dim3(NT), select_lds_bytes(nch), s, p, t);
  else
    hipLaunchKernelGGL(select_chunk_kernel<false>, grid, dim3(NT), select_lds_bytes(nch), s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel

namespace kvsel {

hipError_t launch_select_blocks(const SelectParams &p, const SegTable &t, hipStream_t s) {
  int64_t lmax = 0;
  for (int i = 0; i < t.nseq; ++i) lmax = std::max<int64_t>(lmax, t.key_off[i + 1] - t.key_off[i]);
  const int nch = (int)((lmax + CH - 1) / CH);
  if (nch < 1 || nch > MAXCH) return hipErrorInvalidValue;
  const size_t lds = (size_t)(5 * nch * CPB + 1) * sizeof(int);
  const dim3 grid((unsigned)nch, p.Hkv, t.nseq);
  if (p.K_out)
    hipLaunchKernelGGL(select_block_kernel<true>, dim3(2 * grid.x, grid.y, grid.z), dim3(NT), lds, s, p, t);
  else
    hipLaunchKernelGGL(select_block_kernel<false>, grid, dim3(NT), lds, s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel
