// Two-pass blockwise scoring of every prefix key against the observation rows
// (TideKV, "Delayed KV Eviction via Layer-Wise Chunked Prefill", §4.2).
//
// Work unit: one workgroup of four waves per (key block, KV head, sequence).
// The block's keys are streamed in tiles of 32 keys (8 KiB of K), loaded
// straight from memory into a ring of four LDS slots (global_load_lds, 16
// bytes per lane, each wave a quarter of the tile) three tiles ahead of the
// one being consumed.  The lanes' source chunks are chosen so that a slot
// holds the tile in a swizzled layout (16-byte chunk c of key r sits at
// position c ^ (r & 15) of the row), which makes the MFMA operand reads
// below free of bank conflicts; one barrier per tile lets all four waves
// read it.  The observation rows
// (R = G * w' per KV head, row = window row * G + query head of the group)
// are split into row tiles of 32; wave v owns row tiles v, v+4, v+8, v+12
// and keeps their query fragments in registers for the whole block.
//
// Contraction: v_mfma_f32_32x32x16_bf16 over d = 128 in 8 k-steps.  Lane l
// supplies, at k-step j, the 16-byte chunk 2j + l/32 of row l%32 of each
// operand; the same permutation of the contraction index is used for Q and
// K, so the products are unchanged.
//
// Pass 1 puts the keys in the MFMA's M dimension (A = K, B = Q), so each lane
// holds 16 logits of one observation row.  The lane keeps a reference r and
// Z = sum 2^(x - r) of its base-2 logits x = s * scale * log2(e); r is only
// moved when Z would leave a safe range (checked once per tile for the whole
// wave), so the common path costs one FMA, one exp2 and one add per logit.
// The two lanes of a row are merged with the log-sum-exp rule and each
// block's per-row state is stored; pass 2 starts by combining the
// blocks, in a fixed order, into per row bias = r + log2(Z) - log2(c_r).
//
// Pass 2 puts the observation rows in M (A = Q, B = K), so each lane holds 16
// rows of one key: it adds c_r * p = 2^(x - bias) over its rows in-lane, the
// two lane halves are combined with one swap, the four waves in LDS, in a
// fixed order (no floating-point atomics: results are bit-reproducible).
//
// For kvsel_compress, pass 2 goes on to the selection's first steps over its
// block (TAB): it also scores the kPoolHalo keys past each end of the block
// (one more tile; the same arithmetic in the same order as the block that
// owns them, so the same bits), pools S over the block's positions (TideKV
// §4.2 / DeferKV guide Phase 2 pooling), writes the pooled scores and, per
// kTabBlock positions, counting-sorts the positions by a first digit of
// their order key: the exclusive prefix of the digit histogram, the keys
// grouped by digit, and the histogram added to the segment's.  The
// selection launch finishes the top-k from these tables.  In the streaming
// form the epilogue stops after the pool and writes each pooled score's
// order key, for the running top-k, in place of the tables.
//
// The first digit.  A segment's scores sum to W = G * sum_r c_r, so they
// centre near the mean W / L; the digit counts steps of 2^16 in the order
// key (the fp32 bits, which grow like 2^23 log2 of the value) from the
// mean's key, offset by 1024 and clamped to [0, 2047]: bins of 1/128 of a
// factor 2, 8 factors of 2 either side of the mean.  It is a monotone
// function of the key, so equal values share a bin and higher bins hold
// larger keys, and it leaves a few hundred keys in the bin of the k-th
// largest where a fixed slice of the key's top bits leaves thousands.
#include <atomic>

#include "kvsel_internal.h"
#include "kvsel_device.h"

namespace kvsel {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = kScoreThreads;        // 256 threads, 4 waves
constexpr int NW = NT / 64;
constexpr int KT = kKeyTile;             // 32 keys per tile
constexpr int ROWB = kHeadDim * 2;       // 256 bytes per key row
constexpr int TILE_BYTES = KT * ROWB;    // 8 KiB
static_assert(TILE_BYTES == 2 * 16 * NT, "each thread moves two 16-byte chunks per tile");
// LDS ring slots per pass (tiles in flight = slots - 1).
constexpr int kRing1 = 4;
constexpr int kRing2 = 4;
// s_waitcnt immediate for vmcnt(2 (pd - 2)) with the other counters left alone.
constexpr int wait_tile(int pd) { return 0x3F70 | (2 * (pd - 2)); }
static_assert(kRing1 >= 3 && kRing1 <= 8 && kRing2 >= 3 && kRing2 <= 8, "at most eight named slots; vmcnt fits the low field");

// The LDS ring: one array per slot, so that the compiler can tell a slot
// being read from the slots that loads are landing in (ring(i) is only ever
// called with an index known after unrolling).
#define KVSEL_SLOT(n) __shared__ __attribute__((aligned(16))) char g_ring##n[TILE_BYTES];
KVSEL_SLOT(0) KVSEL_SLOT(1) KVSEL_SLOT(2) KVSEL_SLOT(3) KVSEL_SLOT(4) KVSEL_SLOT(5) KVSEL_SLOT(6) KVSEL_SLOT(7)
#undef KVSEL_SLOT
__device__ __forceinline__ char *ring(int i) {
  switch (i) {
    case 0: return g_ring0;
    case 1: return g_ring1;
    case 2: return g_ring2;
    case 3: return g_ring3;
    case 4: return g_ring4;
    case 5: return g_ring5;
    case 6: return g_ring6;
    default: return g_ring7;
  }
}
constexpr float kZLimit = 0x1p100f;      // a lane's running sum stays below this

__device__ inline bf16x8 as_frag(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

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

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Issues this wave's share of one key tile straight into an LDS slot:
// 16-byte position P = 128 * wave + 64 * i + lane (i = 0, 1) of the slot
// receives chunk (P & 15) ^ (row & 15) of tile row = P >> 4, which leaves
// the slot in the swizzled layout.  kh points at key 0 of this sequence and
// head.  Tile ti of the block [kb0, kb1) holds keys kb0 + 32 ti + row;
// rows past the block re-read its last key, so every load is in bounds (such
// keys are masked or never consumed).  The halo tile (hal) holds key kb1 +
// row (row < HALO) or kb0 - 2 HALO + row, clamped into [0, L - 1] (a clamped
// key's score is never used): each halo key thus sits in the half of the
// tile it has in its own block's tile (key mod 32; block starts are
// multiples of 32), so the split row tile's partial sums land in the same
// waves and S comes out with the same bits.  The two layouts differ only
// in the key index (a select, no branch: the compiler then still knows how
// many loads each wait covers).
__device__ inline void issue_keys(char *slot, const uint16_t *kh, bool hal, int ti, int kb0, int kb1, int L,
                                  int rowstride, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int P = 128 * wave + 64 * i + lane;
    const int row = P >> 4;
    const int kt = min(kb0 + ti * kKeyTile + row, kb1 - 1);
    const int khalo = min(max((row < kPoolHalo) ? kb1 + row : kb0 - 2 * kPoolHalo + row, 0), L - 1);
    const int key = hal ? khalo : kt;
    const uint16_t *src = kh + (int64_t)key * rowstride + (((P & 15) ^ (row & 15)) * 8);
    __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)(slot + (128 * wave + 64 * i) * 16), 16, 0, 0);
  }
}

// Exclusive prefix sum over the workgroup; also returns the total.
__device__ inline int block_exscan(int v, int *tmp, int &total) {
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
  for (int i = 0; i < NW; ++i) {
    const int s = tmp[i];
    before += (i < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// Row bookkeeping: observation row index -> causal limit (last visible key).
__device__ inline int row_limit(int row, const ScoreParams &p, int L) {
  const int r = row / p.G;
  if (!p.causal || r >= p.w) return L - 1;
  return L - p.w + r;  // <= L - 1
}

// x + (the same register of the other lane half), identical in both halves.
__device__ inline float sum_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// x + (the same register of lane l ^ 16), the lane-l value first in lanes
// whose bit 4 is clear (as x + shuffle-xor 16 would add, in the same order
// up to the commutation of one addition).
__device__ inline float sum_rows16(float x) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// The value of x held by lane l ^ 32.
__device__ inline float other_half(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(sw[0]) : __uint_as_float(sw[1]);
}

// Sum of 16 values as four interleaved chains (shorter dependency chains; the
// order is fixed, so results stay reproducible).
__device__ inline float sum16(const float (&e)[16]) {
  const float a = (e[0] + e[4]) + (e[8] + e[12]);
  const float b = (e[1] + e[5]) + (e[9] + e[13]);
  const float c = (e[2] + e[6]) + (e[10] + e[14]);
  const float d = (e[3] + e[7]) + (e[11] + e[15]);
  return (a + b) + (c + d);
}

// log2 of row `row`'s weight c_r (TideKV §4.2 / DeferKV guide Phase 2):
// 1 per window row, 1 - alpha and alpha with a decode row, or the
// normalised exponential weights.
__device__ inline float row_log2_weight(const ScoreParams &p, int row) {
  const int wr = row / p.G;  // observation row: window rows 0 .. w-1, then the decode row
  if (p.weighting == 1) {
    // c_r = 2^(lambda log2(e) (r - r_max)) / norm, relative position r = wr - (w - 1)
    return p.lam2 * (float)(wr - (p.w - 1) - p.has_decode) - p.log2norm;
  }
  float c = 1.0f;
  if (p.has_decode) c = (wr < p.w) ? (1.0f - p.alpha) : p.alpha;
  return (c > 0.0f) ? log2f(c) : -INFINITY;
}

// The start of pass 2: every row's bias = r + log2(Z) - log2(c_r) from the
// segment's nblk pass-1 block states (r, Z).  Two threads per row (row
// row0 + tid / 2, share sh = tid % 2): share sh loads the states of blocks
// sh, sh + 2, ... MB at a time, takes their largest r, m, then the sum of
// Z 2^(r - m) in block order, and folds that into its running state; share
// 0 then takes in share 1.  Every pass-2 workgroup of the segment computes
// the same bits.  The first batch of loads is issued before the key tiles
// (so that waiting for it does not mean waiting for them), by
// MergeRows::load; MergeRows::finish does the rest.  One batch covers 32
// block states (a whole 32K-key prefix in pass 1's blocks of 1024).
struct MergeRows {
  static constexpr int MB = 16;
  float2 v[MB];
  int row, sh;
  const float2 *all;

  // Unconditional loads, clamped into the segment's states (all written by
  // pass 1, so finite or (-inf, 0)); a state past the end becomes (-inf, 0)
  // by arithmetic on the loaded value, which keeps every load outside any
  // branch: loads under a branch would make the compiler wait for every
  // load in flight, the key tiles' too.
  __device__ void load_batch(const ScoreParams &p, int bb0, int nblk) {
    const int rc = min(row, p.Rpad - 1);
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int bb = bb0 + 2 * u;
      const float2 w = all[(int64_t)min(bb, nblk - 1) * p.Rpad + rc];
      const bool ok = bb < nblk && row < p.R;
      v[u] = make_float2(w.x + (ok ? 0.0f : -INFINITY), w.y * (ok ? 1.0f : 0.0f));
    }
  }
  __device__ void fold(float &r, float &z) const {
    float m = v[0].x;
#pragma unroll
    for (int u = 1; u < MB; ++u) m = fmaxf(m, v[u].x);
    if (m > -INFINITY) {
      float t = 0.0f;
#pragma unroll
      for (int u = 0; u < MB; ++u) t = fmaf(v[u].y, fast_exp2(v[u].x - m), t);
      lse_merge(r, z, m, t);
    }
  }
  // The first batch of rows row0 = 0.
  __device__ void load(const ScoreParams &p, int seg, int nblk) {
    all = p.partials + (int64_t)seg * p.nblk1_max * p.Rpad;
    sh = threadIdx.x & 1;
    row = (int)(threadIdx.x >> 1);
    load_batch(p, sh, nblk);
  }
  // The rows of group `row` (its first batch loaded) into out.
  __device__ void group(const ScoreParams &p, int nblk, float *out) {
    float r = -INFINITY, z = 0.0f;
    fold(r, z);
    for (int bb0 = sh + 2 * MB; bb0 < nblk; bb0 += 2 * MB) {
      load_batch(p, bb0, nblk);
      fold(r, z);
    }
    const float r2 = __shfl_xor(r, 1), z2 = __shfl_xor(z, 1);
    if (sh == 0 && row < p.Rpad) {
      lse_merge(r, z, r2, z2);
      const float lc = row_log2_weight(p, row);
      float b = INFINITY;  // a row of weight 0 (or without visible keys) contributes nothing
      if (row < p.R && lc > -INFINITY && z > 0.0f) b = r + log2f(z) - lc;
      out[row] = b;
    }
  }
  // Biases of rows [0, Rpad) into out.  The first group is outside the
  // loop, so that its wait covers only its own loads.
  __device__ void finish(const ScoreParams &p, int nblk, float *out) {
    group(p, nblk, out);
    for (int row0 = NT / 2; row0 < p.Rpad; row0 += NT / 2) {
      row = row0 + (int)(threadIdx.x >> 1);
      load_batch(p, sh, nblk);
      group(p, nblk, out);
    }
  }
};

// The end of pass 2 with tables (see top).  red holds the waves' partial S
// per key (rs floats per wave: the block's keys, then the halo tile's); hist
// and hist1 are 2048 words each of LDS the key ring no longer needs.
__device__ void tables_epilogue(const ScoreParams &p, float *red, int rs, uint32_t *hist, uint32_t *hist1, int seg,
                                int h, int64_t key0, int L, int kb0, int kb1) {
  static_assert(NT == kTabBlock, "one thread per position of a table block");
  static_assert(kTabBins == 8 * NT, "eight bins per thread in the block scan");
  constexpr int HALO = kPoolHalo;
  __shared__ int tmp[NW];
  const int tid = threadIdx.x;
  const int n = kb1 - kb0;
  const int r = p.pool_r;  // 0: no pool
  const bool is_max = p.pool == 2;
  const float fill = is_max ? -INFINITY : 0.0f;  // the pool's value outside the sequence
  float *sbuf = red + NW * rs;                   // S of position kb0 + x at sbuf[HALO + x], x in [-HALO, n + HALO)
  const int64_t segbase = (int64_t)p.Hkv * key0 + (int64_t)h * L;

  // S by position: the sum over the waves in wave order, as pass 2 without
  // tables stores it.
  for (int x = tid - HALO; x < n + HALO; x += NT) {
    const bool in_blk = x >= 0 && x < n;
    if (!in_blk && r == 0) continue;
    const int col = in_blk ? x : p.key_block + ((x < 0) ? 2 * HALO + x : x - n);
    float v = red[col];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) v += red[w2 * rs + col];
    if (in_blk && p.scores) p.scores[segbase + kb0 + x] = v;
    const int pos = kb0 + x;
    if (pos < 0 || pos >= L) v = fill;
    sbuf[HALO + x] = v;
  }
  __syncthreads();

  const uint32_t centre = order_key(p.wsum / (float)L);  // the key of the mean score
  const int ntb = (n + kTabBlock - 1) / kTabBlock;
  uint32_t *hs[2] = {hist, hist1};
  // Two table blocks at a time (tb0, tb0 + 1), thread tid taking position
  // tid of each: their histograms in two LDS arrays, one scan for both.
  for (int tb0 = 0; tb0 < ntb; tb0 += 2) {
    // ---- pool, pooled output
    float P[2];
    int x[2];
    bool ok[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      x[e] = (tb0 + e) * kTabBlock + tid;
      ok[e] = x[e] < n;  // (past the last table block: x >= n)
      P[e] = 0.0f;
      if (ok[e]) {
        const float *c = sbuf + HALO + x[e];
        if (r == 0) {
          P[e] = c[0];
        } else if (is_max) {
          float m = c[0];
          for (int j = -r; j <= r; ++j) m = fmaxf(m, c[j]);
          P[e] = m;
        } else {
          float sum = 0.0f;
          for (int j = -r; j <= r; ++j) sum += c[j];
          P[e] = sum / p.pool_width;
        }
        if (p.pooled) p.pooled[segbase + kb0 + x[e]] = P[e];
      }
    }
    if (p.step_keys) {
      // the streaming form: the pooled scores' order keys, no tables
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (ok[e])
          p.step_keys[(int64_t)seg * p.step_stride + (kb0 + x[e] - p.step_origin)] =
              select_key(P[e], kb0 + x[e], L, p.sink, p.recent);
      continue;
    }

    // ---- counting sort of each table block by first digit; the segment
    // histogram
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      reinterpret_cast<uint4 *>(hs[e])[2 * tid] = make_uint4(0u, 0u, 0u, 0u);
      reinterpret_cast<uint4 *>(hs[e])[2 * tid + 1] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    uint32_t key[2], dg[2], rank[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      key[e] = 0u;
      dg[e] = 0u;
      rank[e] = 0u;
      if (ok[e]) {
        key[e] = select_key(P[e], kb0 + x[e], L, p.sink, p.recent);
        const int64_t rel = ((int64_t)key[e] - (int64_t)centre) >> kTabDigitShift;
        dg[e] = (uint32_t)min<int64_t>(kTabBins - 1, max<int64_t>(0, rel + kTabBins / 2));
        rank[e] = atomicAdd(&hs[e][dg[e]], 1u);
      }
    }
    __syncthreads();
    uint32_t cnt[2][8], pre[2][8];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint4 a0 = reinterpret_cast<const uint4 *>(hs[e])[2 * tid];
      const uint4 a1 = reinterpret_cast<const uint4 *>(hs[e])[2 * tid + 1];
      cnt[e][0] = a0.x; cnt[e][1] = a0.y; cnt[e][2] = a0.z; cnt[e][3] = a0.w;
      cnt[e][4] = a1.x; cnt[e][5] = a1.y; cnt[e][6] = a1.z; cnt[e][7] = a1.w;
    }
    int own = 0;  // both blocks' counts in this thread's bins, 16 bits each (at most 256)
#pragma unroll
    for (int u = 0; u < 8; ++u) own += (int)(cnt[0][u] | (cnt[1][u] << 16));
    int total;
    const int ex = block_exscan(own, tmp, total);  // its barriers end the reads above
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint32_t run = (uint32_t)(ex >> (16 * e)) & 0xffffu;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pre[e][u] = run;
        run += cnt[e][u];
      }
      if (tb0 + e < ntb) {
        const int64_t tabi = (int64_t)seg * p.ntab_max + kb0 / kTabBlock + tb0 + e;
        reinterpret_cast<uint4 *>(p.tab + tabi * kTabBins)[tid] =
            make_uint4(pre[e][0] | (pre[e][1] << 16), pre[e][2] | (pre[e][3] << 16), pre[e][4] | (pre[e][5] << 16),
                       pre[e][6] | (pre[e][7] << 16));
      }
    }
    // this workgroup's copy of the segment histogram: consecutive
    // workgroups go to different compute dies, and so do the copies
    const int copy = (int)((blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)) % kTabHistCopies);
    uint32_t *shc = p.seg_hist + ((int64_t)seg * kTabHistCopies + copy) * kTabBins + 8 * tid;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t cu = cnt[0][u] + cnt[1][u];
      if (cu) atomicAdd(shc + u, cu);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      reinterpret_cast<uint4 *>(hs[e])[2 * tid] = make_uint4(pre[e][0], pre[e][1], pre[e][2], pre[e][3]);
      reinterpret_cast<uint4 *>(hs[e])[2 * tid + 1] = make_uint4(pre[e][4], pre[e][5], pre[e][6], pre[e][7]);
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (ok[e]) {
        const int64_t tabi = (int64_t)seg * p.ntab_max + kb0 / kTabBlock + tb0 + e;
        p.bucket[tabi * kTabBlock + hs[e][dg[e]] + rank[e]] = key[e];
      }
    }
    __syncthreads();  // the histograms are cleared for the next pair
  }
}

// RT: full row tiles (of 32 rows) per wave.  SPLIT: there is one more row
// tile (4 RT + 1 in all), split into four 16 x 16 blocks per key tile, one
// per wave: wave v takes its rows 16 (v / 2) .. + 15 against the key tile's
// keys 16 (v % 2) .. + 15, with v_mfma_f32_16x16x32_bf16, so that no wave
// carries a whole extra tile (the slowest wave sets every step's pace).
// TAB (pass 2 only): the halo tile, pool and selection tables (see top).
// The waves per SIMD the registers are planned for: pass 2 with tables and
// one whole row tile per wave fits three (168 VGPRs), so that three
// workgroups share a compute unit and one's prologue and epilogue overlap
// the others' key streams (measured faster than two); pass 2 otherwise two;
// pass 1 with one whole row tile per wave two (room for PIPE's second
// accumulator set), else as the row tiles allow.
template <int PASS, int RT, bool SPLIT = false, bool TAB = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu((PASS == 1 && RT == 1 && !SPLIT) ? 2 : (PASS == 2 && RT == 1) ? ((TAB && !SPLIT) ? 3 : 2) : SPLIT ? (RT > 2 ? 1 : 2) : RT > 1 ? 1 : 4))) void score_kernel(ScoreParams p, SegTable t) {
  extern __shared__ float red[];  // pass 2: [NW][rs] partial sums (TAB: then S by position)
  constexpr int PD = (PASS == 1) ? kRing1 : kRing2;  // LDS ring slots
  constexpr int kWaitTile = wait_tile(PD);

  const int blk = blockIdx.x;
  const int h = blockIdx.y;
  const int sb = blockIdx.z;
  // Launches of two workgroups per compute unit (pass 2 with the pool; pass
  // 1 with two row tiles per wave or a split one): the workgroup dispatched
  // first wins the issue arbitration (older waves go first), and the second
  // finished about 4 us later on a 32K-key Llama-shaped layer, alone on the
  // unit for that time.  The second ones (linear index in [young_from,
  // 2 young_from)) take a higher priority for the first half of their key
  // tiles, which evens the two out.  Only where it measured faster: the
  // check in the loop cost pass 1 with one whole row tile per wave (one
  // workgroup per unit there) 2%.
  constexpr bool PRIO = (PASS == 2 && TAB) || RT > 1 || SPLIT;
  const int wg_lin = blk + (int)gridDim.x * (h + (int)gridDim.y * sb);
  const bool young = PRIO && p.young_from > 0 && wg_lin >= p.young_from && wg_lin < 2 * p.young_from;
  if (young) __builtin_amdgcn_s_setprio(1);
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  // Keys key_begin + blk * key_block onwards, clipped to [key_begin,
  // key_end) of the launch (the whole prefix unless streaming).
  const int kend = min(L, p.key_end);
  const int kb0 = p.key_begin + blk * p.key_block;
  if (kb0 >= kend) return;  // the whole workgroup leaves together
  const int kb1 = min(kend, kb0 + p.key_block);
  const int seg = t.seg0 + sb * p.Hkv + h;
  if (PASS == 1 && p.seg_hist) {
    // this block's slice of the segment's selection histogram (all its
    // copies), cleared for the pass 2 that adds to it
    constexpr int nw = kTabHistCopies * kTabBins;
    const int nbs = (L + p.key_block - 1) / p.key_block;
    const int z0 = (int)((int64_t)blk * nw / nbs), z1 = (int)((int64_t)(blk + 1) * nw / nbs);
    for (int i = z0 + (int)threadIdx.x; i < z1; i += NT) p.seg_hist[(int64_t)seg * nw + i] = 0u;
  }
  const int b = t.seq0 + sb;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31;  // row (pass 1: observation row; pass 2: key) within a 32-tile
  const int hf = lane >> 5;  // lane half: chunk parity, and rows 4*hf.. of the output
  const int nrt = p.nrt;     // row tiles of 32 over all waves
  int my_rt = 0;             // row tiles this wave owns (wave-uniform)
#pragma unroll
  for (int k = 0; k < RT; ++k) my_rt += (wave + NW * k < nrt) ? 1 : 0;

  // Query fragments of this wave's row tiles: lane supplies row lr of the
  // tile, chunks 2j + hf.
  bf16x8 qf[RT][8];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    const int row = (wave + NW * k) * 32 + lr;
    if (k < my_rt && row < p.R) {
      const int r = row / p.G;
      const int gi = row - r * p.G;
      const uint16_t *src = p.Q + ((int64_t)(b * p.wp + r) * p.Hq + h * p.G + gi) * (int64_t)kHeadDim + hf * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[k][j] = as_frag(*reinterpret_cast<const uint4 *>(src + 16 * j));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[k][j] = as_frag(make_uint4(0u, 0u, 0u, 0u));
    }
  }

  // Per-lane state.  Pass 1: reference, sum and causal limit of the lane's
  // row in each row tile.  Pass 2: bias of the lane's 16 rows per row tile.
  float ref[RT], zs[RT];
  int lim[RT];
  float bias[RT][16];
#pragma unroll
  for (int k = 0; k < RT; ++k) {
    ref[k] = -INFINITY;
    zs[k] = 0.0f;
    // pass 1: a key past the block's end (a re-read of its last key) is
    // masked like a key past the row's causal limit
    lim[k] = min(row_limit((wave + NW * k) * 32 + lr, p, L), kb1 - 1);
  }

  // The split tile.  Lane l supplies, at k-step j (32 wide), row (or key)
  // l % 16 of its block and the 16-byte chunk 4 j + l / 16 of it; the
  // output holds entries 4 (l / 16) + i (i < 4) of the block's first
  // operand against entry l % 16 of the second.  Pass 1: A = keys, B = rows,
  // so a lane holds 4 keys of one row (sr); pass 2: A = rows, B = keys, so a
  // lane holds 4 rows (sr4 + i) of one key.
  const int s16 = lane & 15, s4 = lane >> 4;
  const int srow = NW * RT * 32 + 16 * (wave >> 1);  // first row of this wave's block
  const int skey = 16 * (wave & 1);                  // first key of this wave's block in a key tile
  bf16x8 qs[4];
  float ref5 = -INFINITY, zs5 = 0.0f, bias5[4];
  int lim5r[4] = {0, 0, 0, 0};  // pass 2: the split rows' causal limits
  int lim5 = 0;
  if constexpr (SPLIT) {
    const int row = srow + s16;
    if (row < p.R) {
      const int r = row / p.G;
      const int gi = row - r * p.G;
      const uint16_t *src = p.Q + ((int64_t)(b * p.wp + r) * p.Hq + h * p.G + gi) * (int64_t)kHeadDim + s4 * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) qs[j] = as_frag(*reinterpret_cast<const uint4 *>(src + 32 * j));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) qs[j] = as_frag(make_uint4(0u, 0u, 0u, 0u));
    }
    lim5 = min(row_limit(row, p, L), kb1 - 1);
  }
  // LDS byte offsets of this lane's split-tile key operand at k-step j: key
  // skey + s16 of the tile, chunk 4 j + s4, swizzled like the 32-wide reads.
  int srd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = skey + s16;
    srd[j] = kr * ROWB + (((4 * j + s4) ^ (kr & 15)) << 4);
  }

  const float cl2 = p.cl2;
  const int minlim = p.causal ? (L - p.w) : (L - 1);  // keys up to here are visible to every row
  const int ntile = (kb1 - kb0 + KT - 1) / KT;
  // TAB with a pool: one more step scores the halo tile (its keys after the
  // block's in red: rs floats per wave).
  const bool halo = TAB && p.pool_r > 0;
  const int nsteps = ntile + (halo ? 1 : 0);
  const int rs = TAB ? p.key_block + 2 * kPoolHalo : p.key_block;
  const int rowstride = p.Hkv * kHeadDim;  // elements between consecutive keys of one head
  // LDS byte offset of this lane's operand chunk for k-step j: row lr, chunk 2j + hf, swizzled.
  const int rd_base = lr * ROWB;
  const int sw = lr & 15;

  // Tiles go straight from memory into a ring of PD LDS slots, PD - 1
  // tiles ahead of the one being consumed.  Every step issues exactly two
  // loads per wave (past the block they re-read its last key), so before
  // step t this wave has tiles t .. t + PD - 2 in flight, and waiting until
  // at most 2 (PD - 2) loads remain means tile t has landed.
  const uint16_t *kh = p.K + key0 * (int64_t)rowstride + (int64_t)h * kHeadDim;
  auto issue = [&](char *slot, int ti) { issue_keys(slot, kh, halo && ti == ntile, ti, kb0, kb1, L, rowstride, wave, lane); };
  MergeRows mr;
  const int nstat = (int)((L + (int64_t)p.stat_block - 1) / p.stat_block);  // pass-1 block states per row
  if constexpr (PASS == 2) mr.load(p, seg, nstat);
#pragma unroll
  for (int j = 0; j < PD - 1; ++j) issue(ring(j), j);

  if constexpr (PASS == 2) {
    // The row biases, merged while the first tiles load.
    __shared__ float bias_s[kMaxRows];
    mr.finish(p, nstat, bias_s);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < RT; ++k) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = (wave + NW * k) * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
        bias[k][i] = (k < my_rt) ? bias_s[row] : INFINITY;
      }
    }
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bias5[i] = bias_s[srow + 4 * s4 + i];
        lim5r[i] = row_limit(srow + 4 * s4 + i, p, L);  // the split rows' causal limits
      }
    }
  }

  // Two stages per key tile: its MFMAs (reading the tile from its LDS slot)
  // and its exp / sum work on the accumulators.  With PIPE, step t issues
  // tile t's MFMAs and then does tile t - 1's exp / sum work, which depends
  // only on registers, so the wave's VALU work runs while its matrix core
  // works (two accumulator sets alternate); without PIPE both stages of
  // tile t run in step t.  PIPE is used where it measured faster: one row
  // tile per wave and no split tile (pass 1's registers are then planned for
  // two waves per SIMD); with two row tiles per wave, or a split tile, it is
  // slower.
  constexpr bool PIPE = RT == 1 && !SPLIT;
  static_assert(!PIPE || PD % 2 == 0, "accumulator sets alternate with the slot parity");
  f32x16 accs[PIPE ? 2 : 1][RT];
  f32x4 saccs[PIPE ? 2 : 1];

  auto mfma_tile = [&](const char *slot, f32x16 (&acc)[RT], f32x4 &sacc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8 kf = as_frag(*reinterpret_cast<const uint4 *>(slot + rd_base + (((2 * j + hf) ^ sw) << 4)));
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        if (k < my_rt) {
          const f32x16 c = (j == 0) ? f32x16{} : acc[k];
          if constexpr (PASS == 1)
            acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[k][j], c, 0, 0, 0);
          else
            acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[k][j], kf, c, 0, 0, 0);
        }
      }
    }
    sacc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (SPLIT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 kf = as_frag(*reinterpret_cast<const uint4 *>(slot + srd[j]));
        if constexpr (PASS == 1)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qs[j], sacc, 0, 0, 0);
        else
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qs[j], kf, sacc, 0, 0, 0);
      }
    }
  };

  // The exp / sum stage of tile ti from its accumulators.
  auto valu_tile = [&](const int ti, const f32x16 (&acc)[RT], const f32x4 &sacc) {
    const int i0 = kb0 + ti * KT;
    // The halo step: key x of the tile is kb1 + x or kb0 - 2 HALO + x.
    const bool hstep = halo && ti == ntile;
    auto key_at = [&](int x) { return hstep ? ((x < kPoolHalo) ? kb1 + x : kb0 - 2 * kPoolHalo + x) : i0 + x; };
    const int rbase = wave * rs + (hstep ? p.key_block : ti * KT);  // this tile's keys in red
    if (my_rt == 0) {  // this wave owns no rows (fewer than four row tiles in all)
      if constexpr (PASS == 2)
        if (hf == 0) red[rbase + lr] = 0.0f;
      return;
    }
    const bool need_mask = hstep || (i0 + KT - 1) > ((PASS == 1) ? min(minlim, kb1 - 1) : minlim);

    if constexpr (PASS == 1) {
      // acc[k][i]: key i0 + 8*(i/4) + 4*hf + i%4, row of this lane.
      bool bad = false;
      float znew[RT];
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        float e[16];
        if (!need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) e[i] = fast_exp2(fmaf(acc[k][i], cl2, -ref[k]));
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float v = fast_exp2(fmaf(acc[k][i], cl2, -ref[k]));
            e[i] = ((i0 + 8 * (i >> 2) + 4 * hf + (i & 3)) > lim[k]) ? 0.0f : v;
          }
        }
        // Row tiles this wave does not own skipped their MFMAs: their
        // accumulators hold stale register contents and must not be summed.
        znew[k] = (k < my_rt) ? zs[k] + sum16(e) : 0.0f;
        bad |= (k < my_rt) && !(znew[k] <= kZLimit);
      }
      // sacc[i]: key i0 + skey + 4 s4 + i, row srow + s16.
      float znew5 = 0.0f;
      if constexpr (SPLIT) {
        float e5[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = fast_exp2(fmaf(sacc[i], cl2, -ref5));
          e5[i] = (need_mask && (i0 + skey + 4 * s4 + i) > lim5) ? 0.0f : v;
        }
        znew5 = zs5 + ((e5[0] + e5[1]) + (e5[2] + e5[3]));
        bad |= !(znew5 <= kZLimit);
      }
      if (__builtin_expect(__ballot(bad) != 0ull, 0)) {
        if constexpr (SPLIT) {
          float m = ref5;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!need_mask || (i0 + skey + 4 * s4 + i) <= lim5) m = fmaxf(m, sacc[i] * cl2);
          float z = (ref5 == -INFINITY || m == -INFINITY) ? 0.0f : zs5 * fast_exp2(ref5 - m);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!need_mask || (i0 + skey + 4 * s4 + i) <= lim5) z += fast_exp2(fmaf(sacc[i], cl2, -m));
          ref5 = m;
          zs5 = z;
        }
        // Rare (always on a wave's first tile): move each reference up to
        // the largest logit seen so far and redo this tile's sum.
#pragma unroll
        for (int k = 0; k < RT; ++k) {
          if (k >= my_rt) continue;
          float m = ref[k];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const bool vis = !need_mask || (i0 + 8 * (i >> 2) + 4 * hf + (i & 3)) <= lim[k];
            if (vis) m = fmaxf(m, acc[k][i] * cl2);
          }
          float z = (ref[k] == -INFINITY || m == -INFINITY) ? 0.0f : zs[k] * fast_exp2(ref[k] - m);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const bool vis = !need_mask || (i0 + 8 * (i >> 2) + 4 * hf + (i & 3)) <= lim[k];
            if (vis) z += fast_exp2(fmaf(acc[k][i], cl2, -m));
          }
          ref[k] = m;
          zs[k] = z;
        }
      } else {
#pragma unroll
        for (int k = 0; k < RT; ++k) zs[k] = znew[k];
        if constexpr (SPLIT) zs5 = znew5;
      }
    } else {
      // acc[k][i]: row 8*(i/4) + 4*hf + i%4 of row tile k, key i0 + lr.
      float part[RT];
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        float e[16];
        if (!need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) e[i] = fast_exp2(fmaf(acc[k][i], cl2, -bias[k][i]));
        } else {
          const int key = key_at(lr);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row = (wave + NW * k) * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
            const float v = fast_exp2(fmaf(acc[k][i], cl2, -bias[k][i]));
            e[i] = (key > row_limit(row, p, L)) ? 0.0f : v;
          }
        }
        part[k] = (k < my_rt) ? sum16(e) : 0.0f;  // unowned tiles: stale accumulators
      }
      float s = part[0];
#pragma unroll
      for (int k = 1; k < RT; ++k) s += part[k];
      s = sum_halves(s);
      if constexpr (SPLIT) {
        // sacc[i]: row srow + 4 s4 + i, key i0 + skey + s16.  Sum the rows,
        // then over the four lane groups: every lane then holds the block's
        // sum for key skey + s16, which lane lr adds when that is its key.
        float s5 = 0.0f;
        if (!need_mask) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s5 += fast_exp2(fmaf(sacc[i], cl2, -bias5[i]));
        } else {
          const int key5 = key_at(skey + s16);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = fast_exp2(fmaf(sacc[i], cl2, -bias5[i]));
            s5 += (key5 > lim5r[i]) ? 0.0f : v;
          }
        }
        s5 = sum_halves(sum_rows16(s5));
        s += ((lr >> 4) == (wave & 1)) ? s5 : 0.0f;
      }
      if (hf == 0) red[rbase + lr] = s;
    }
  };

  // Step ti: waits for tile ti, refills the slot of tile ti - 1 with tile
  // ti + PD - 1, then runs the stages due (j: ti mod PD, known after
  // unrolling).
  auto step = [&](const int ti, const int j, const char *cur, char *nxt) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(kWaitTile);  // this wave's part of tile ti is in LDS
    __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): this wave's reads of tile ti - 1 are done
    __builtin_amdgcn_s_barrier();           // every wave's part has landed; nxt is free
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    issue(nxt, ti + PD - 1);
    if constexpr (PIPE) {
      if (ti < nsteps && my_rt > 0) mfma_tile(cur, accs[j & 1], saccs[j & 1]);
      if (ti >= 1 && ti <= nsteps) valu_tile(ti - 1, accs[(j + 1) & 1], saccs[(j + 1) & 1]);
    } else {
      if (ti < nsteps) {
        if (my_rt > 0) mfma_tile(cur, accs[0], saccs[0]);
        valu_tile(ti, accs[0], saccs[0]);
      }
    }
  };
  const int nloop = PIPE ? nsteps + 1 : nsteps;  // PIPE: one more step for the last tile's exp / sum
  for (int t0 = 0; t0 < nloop; t0 += PD) {
    if (young && t0 == ((nloop / 2) & ~(PD - 1))) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < PD; ++j) step(t0 + j, j, ring(j), ring((j + PD - 1) % PD));
  }
  // The last steps issued loads for tiles past the block that nobody
  // consumes; they write LDS, so drain them before the workgroup can end.
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  if constexpr (PASS == 2 && TAB) {
    __syncthreads();
    tables_epilogue(p, red, rs, reinterpret_cast<uint32_t *>(g_ring0), reinterpret_cast<uint32_t *>(g_ring1), seg, h,
                    key0, L, kb0, kb1);
  } else if constexpr (PASS == 2) {
    __syncthreads();
    const int n = kb1 - kb0;
    // The public layout, or (streaming) one window of out_stride floats per
    // segment whose first element is key out_origin.
    float *out = (p.out_stride > 0) ? p.scores + (int64_t)seg * p.out_stride + (kb0 - p.out_origin)
                                    : p.scores + (int64_t)p.Hkv * key0 + (int64_t)h * L + kb0;
    for (int i = threadIdx.x; i < n; i += NT) {
      float v = red[i];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) v += red[w2 * p.key_block + i];
      out[i] = v;
    }
  } else {
    // Merge the two lane halves that share each row and publish this
    // block's per-row state; pass 2 merges the blocks.
    float2 *part = p.partials + ((int64_t)seg * p.nblk1_max + blk) * p.Rpad;
#pragma unroll
    for (int k = 0; k < RT; ++k) {
      const float r2 = other_half(ref[k]);
      const float z2 = other_half(zs[k]);
      lse_merge(ref[k], zs[k], r2, z2);
      const int row = (wave + NW * k) * 32 + lr;
      if (hf == 0 && k < my_rt) part[row] = make_float2(ref[k], zs[k]);
    }
    if constexpr (SPLIT) {
      // The four lanes of a row (s4 = 0..3), then the two waves of a row
      // half (their key halves), in a fixed order.
      float r2 = __shfl_xor(ref5, 16), z2 = __shfl_xor(zs5, 16);
      lse_merge(ref5, zs5, r2, z2);
      r2 = __shfl_xor(ref5, 32);
      z2 = __shfl_xor(zs5, 32);
      lse_merge(ref5, zs5, r2, z2);
      __shared__ float2 xchg[NW / 2][16];
      if ((wave & 1) && s4 == 0) xchg[wave >> 1][s16] = make_float2(ref5, zs5);
      __syncthreads();
      if (!(wave & 1) && s4 == 0) {
        const float2 o = xchg[wave >> 1][s16];
        lse_merge(ref5, zs5, o.x, o.y);
        part[srow + s16] = make_float2(ref5, zs5);
      }
    }
  }
}

// The streaming form's fold (TideKV §4.2 with a bounded workspace): the
// block states of the step's keys [key_begin, key_end) merged, in a fixed
// order, into the running state `run` of each row (its first step starts
// it); the fused streaming form merges all of a segment's block states at
// once this way, so that its steps' pass 2 each read one state per row.
// Workgroup (row group of 16, segment): sixteen threads share a row,
// each merging every sixteenth block with 16 loads in flight; the shares
// are combined in a fixed order through LDS.
constexpr int MERGE_ROWS = 16;
constexpr int MERGE_SPLIT = NT / MERGE_ROWS;

__global__ __launch_bounds__(NT) void fold_kernel(ScoreParams p, SegTable t, float2 *run, int first) {
  __shared__ float2 shares[MERGE_SPLIT][MERGE_ROWS];
  const int sl = blockIdx.y;  // local segment: sequence-major, head-minor
  const int sb = sl / p.Hkv;
  const int seg = t.seg0 + sl;
  const int L = (int)(t.key_off[sb + 1] - t.key_off[sb]);
  const int kend = min(L, p.key_end);
  const int nblk = (kend > p.key_begin) ? (kend - p.key_begin + p.key_block - 1) / p.key_block : 0;
  const int lrow = threadIdx.x % MERGE_ROWS;
  const int sh = threadIdx.x / MERGE_ROWS;
  const int row = blockIdx.x * MERGE_ROWS + lrow;
  const float2 *all = p.partials + (int64_t)seg * p.nblk1_max * p.Rpad;
  float r = -INFINITY, z = 0.0f;
  if (row < p.R) {
    for (int bb0 = sh; bb0 < nblk; bb0 += 16 * MERGE_SPLIT) {
      float2 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int bb = bb0 + u * MERGE_SPLIT;
        v[u] = (bb < nblk) ? all[(int64_t)bb * p.Rpad + row] : make_float2(-INFINITY, 0.0f);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) lse_merge(r, z, v[u].x, v[u].y);
    }
  }
  shares[sh][lrow] = make_float2(r, z);
  __syncthreads();
  if (sh != 0 || row >= p.Rpad) return;
#pragma unroll
  for (int k = 1; k < MERGE_SPLIT; ++k) lse_merge(r, z, shares[k][lrow].x, shares[k][lrow].y);
  float2 *mine = run + (int64_t)seg * p.Rpad + row;
  if (!first) {
    const float2 prev = *mine;
    lse_merge(r, z, prev.x, prev.y);
  }
  *mine = make_float2(r, z);
}

template <int PASS, bool TAB = false>
hipError_t launch_pass(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s, size_t lds) {
  const dim3 grid(nblk, p.Hkv, t.nseq);
  const dim3 block(NT);
  if (p.nrt % NW == 1 && p.nrt > NW) {  // whole row tiles per wave plus a split one
    switch (p.nrt / NW) {
      case 1: hipLaunchKernelGGL((score_kernel<PASS, 1, true, TAB>), grid, block, lds, s, p, t); break;
      case 2: hipLaunchKernelGGL((score_kernel<PASS, 2, true, TAB>), grid, block, lds, s, p, t); break;
      default: hipLaunchKernelGGL((score_kernel<PASS, 3, true, TAB>), grid, block, lds, s, p, t); break;
    }
    return hipGetLastError();
  }
  const int rt = (p.nrt + NW - 1) / NW;
  switch (rt) {
    case 1: hipLaunchKernelGGL((score_kernel<PASS, 1, false, TAB>), grid, block, lds, s, p, t); break;
    case 2: hipLaunchKernelGGL((score_kernel<PASS, 2, false, TAB>), grid, block, lds, s, p, t); break;
    case 3: hipLaunchKernelGGL((score_kernel<PASS, 3, false, TAB>), grid, block, lds, s, p, t); break;
    default: hipLaunchKernelGGL((score_kernel<PASS, 4, false, TAB>), grid, block, lds, s, p, t); break;
  }
  return hipGetLastError();
}

}  // namespace

// The compute units of the current device (cached per device; 0 if unknown).
static int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) n = 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_score_pass1(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  ScoreParams q = p;
  q.young_from = compute_units();
  return launch_pass<1>(q, t, nblk, s, 0);
}

hipError_t launch_stream_stats(const ScoreParams &p, const SegTable &t, float2 *run, int first, hipStream_t s) {
  const dim3 grid((p.Rpad + MERGE_ROWS - 1) / MERGE_ROWS, t.nseq * p.Hkv);
  hipLaunchKernelGGL(fold_kernel, grid, dim3(NT), 0, s, p, t, run, first);
  return hipGetLastError();
}

hipError_t launch_score_pass2(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  ScoreParams q = p;
  q.young_from = compute_units();
  return launch_pass<2>(q, t, nblk, s, (size_t)NW * p.key_block * sizeof(float));
}

hipError_t launch_score_pass2_tables(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  if (p.key_block % kTabBlock != 0 || p.pool_r < 0 || p.pool_r > kPoolHalo || !p.pooled || !p.tab || !p.bucket ||
      !p.seg_hist || p.step_keys)
    return hipErrorInvalidValue;
  const size_t rs = (size_t)p.key_block + 2 * kPoolHalo;
  ScoreParams q = p;
  q.young_from = compute_units();
  return launch_pass<2, true>(q, t, nblk, s, (NW + 1) * rs * sizeof(float));
}

hipError_t launch_score_pass2_keys(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  if (p.key_block <= 0 || p.key_block % kKeyTile != 0 || p.pool_r < 0 || p.pool_r > kPoolHalo || !p.step_keys ||
      p.tab || p.pooled || p.scores || p.step_stride <= 0)
    return hipErrorInvalidValue;
  const size_t rs = (size_t)p.key_block + 2 * kPoolHalo;
  ScoreParams q = p;
  q.young_from = compute_units();
  return launch_pass<2, true>(q, t, nblk, s, (NW + 1) * rs * sizeof(float));
}

}  // namespace kvsel
