// Fused scoring: TideKV's two-pass blockwise procedure ("Delayed KV Eviction
// via Layer-Wise Chunked Prefill", §4.2) in one launch, with each key read
// from memory once and each exponential computed once.
//
// Work unit: one workgroup of four waves per block of 256 keys of one
// (sequence, KV head) segment; two such workgroups share a compute unit, so
// one's waits overlap the other's arithmetic.  The block's keys (64 KiB,
// plus a halo tile for the pool) are loaded straight from memory into LDS
// (global_load_lds, 16 bytes per lane, every tile's loads issued up front).
//
//  1. Pass 1: the logits of the block against the segment's observation
//     rows.  For every (row, key) the lane keeps e = 2^(x - ref_row) in
//     registers, where x = s * scale * log2(e) and ref_row is the row's
//     largest logit in the block's first tile, and the row's block sum
//     Z = sum of e.  Published per row: log2 of the block's sum, ref + log2 Z.
//  2. The segment's first block waits until every block has published,
//     merges the per-block results into each row's normaliser and weight,
//     bias_r = log2(sum over blocks) - log2(c_r), and publishes the biases;
//     the other blocks wait for them.
//  3. Pass 2 without recomputing anything: the normalised, weighted
//     probability of (row, key) is e * 2^(ref_row - bias_row), so each key's
//     score S = sum over the group's rows (TideKV §4.2 aggregation; DeferKV
//     guide, Phase 2 row weights) is one FMA per row.  Only the halo tile
//     (16 keys each side of the block, for the pool) takes the MFMA and the
//     exponential again.
//  4. The 1-D pool of the block's positions, the pooled scores written out,
//     and the block's counting sort by a first digit of each pooled value's
//     order key: the exclusive prefix of the block's digit histogram, the
//     keys grouped by digit, and the histogram added to the segment's.  The
//     selection kernel finishes the top-k from these.
//
// Overflow: e stays below 2^100 as long as no logit of a row exceeds that
// row's first-tile maximum by 100 (in log2 units).  A wave whose block sums
// go past that bound (or are not finite) finds each row's true maximum over
// the block first and computes e again, so e <= 1.
//
// The first digit.  A segment's scores sum to W = G * sum_r c_r, so they
// centre near the mean W / L; the digit counts steps of 2^16 in the order
// key (the fp32 bits, which grow like 2^23 log2 of the value) from the
// mean's key, offset by 1024 and clamped to [0, 2047]: bins of 1/128 of an
// octave, 8 octaves either side of the mean.  It is a monotone function of
// the key, so equal values share a bin and higher bins hold larger keys,
// and it leaves a few hundred keys in the bin of the k-th largest where a
// fixed slice of the key's top bits leaves thousands (the scores of a
// segment cluster within a fraction of an octave).
//
// Waiting on other workgroups.  A segment's blocks are consecutive
// workgroups, which start together.  A block publishes its row results,
// then a flag holding this call's token (one more than the token the
// previous call saw, so flags left by earlier calls never match and nothing
// needs clearing).  Every wait is bounded: after spin_cap polls a block
// computes pass 1 of the blocks that have not published yet itself (the
// same code on the same keys, so the same bits) and merges on its own, so
// the kernel ends whatever else shares the GPU and in whatever order its
// workgroups run.  Such a block leaves the segment's histogram alone and
// marks it incomplete (the selection then rebuilds it from the blocks'
// tables).  Before publishing, every block clears its slice of the segment
// histogram, so the histogram is clear before any block that saw all flags
// adds to it.  Cross-workgroup data moves with device-scope atomic loads
// and stores (coherent across the chip's L2s without cache write-backs); a
// block's results are complete before its flag is set.
//
// Rows: the R = G * w' <= 128 observation rows of the KV head (row = window
// row * G + query head of the group) are split into row tiles of 32; wave v
// owns row tile v over every key tile.  Contraction: v_mfma_f32_32x32x16_bf16
// over d = 128 in 8 k-steps, rows in the first operand and keys in the
// second, so a lane holds 16 rows (8 (i / 4) + 4 (l / 32) + i % 4) of one
// key (l % 32); lane l supplies, at k-step j, the 16-byte chunk 2 j + l / 32
// of entry l % 32 of each operand (the same permutation of the contraction
// index on both operands leaves the products unchanged).
#include <algorithm>

#include "kvsel_internal.h"
#include "kvsel_device.h"

namespace kvsel {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NT = kResThreads;        // 256 threads
constexpr int NW = NT / 64;            // 4 waves
constexpr int KT = kKeyTile;           // 32 keys per tile
constexpr int BLK = kResBlock;         // 256 keys per workgroup
constexpr int NTILE = BLK / KT;        // 8 tiles
constexpr int ROWB = kHeadDim * 2;     // 256 bytes per key row
constexpr int TILE_BYTES = KT * ROWB;  // 8 KiB
constexpr int HALO = kResHalo;         // 16
constexpr int SIDX = BLK + 2 * HALO;   // per-row-tile key sums: block keys, then the halo tile's
constexpr int NBIN = kResBins;         // 2048
constexpr int DSHIFT = kResDigitShift; // 16
constexpr float kZLimit = 0x1p100f;
static_assert(TILE_BYTES == 2 * NT * 16, "two 16-byte chunks per lane and tile");
static_assert(NT == BLK, "one thread per position of a block in the epilogue");
static_assert(NBIN == 8 * NT, "eight bins per thread in the block scan");
static_assert(NBIN == 2048, "digits centre on bin 1024");
static_assert(kResMaxRows == NW * 32, "one row tile of 32 per wave");

// The block's key tiles in LDS, two per array: an unrolled step names its
// pair's array, so the compiler waits only for that pair's loads (an array
// it cannot tell apart from the others would make it wait for all of them).
#define KVSEL_PAIR(n) __shared__ __attribute__((aligned(16))) char g_pair##n[2 * TILE_BYTES];
KVSEL_PAIR(0) KVSEL_PAIR(1) KVSEL_PAIR(2) KVSEL_PAIR(3)
#undef KVSEL_PAIR
__shared__ __attribute__((aligned(16))) char g_halo[TILE_BYTES];

__device__ __forceinline__ char *pair_at(int i) {
  switch (i) {
    case 0: return g_pair0;
    case 1: return g_pair1;
    case 2: return g_pair2;
    default: return g_pair3;
  }
}

// Key tile t (0 .. 7), or the halo tile (t = 8).
__device__ __forceinline__ char *tile_at(int t) {
  return (t >= NTILE) ? g_halo : pair_at(t >> 1) + (t & 1) * TILE_BYTES;
}

__device__ inline bf16x8 as_frag(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left alone.
constexpr int vm_wait(int n) { return 0x3F70 | (n & 15) | ((n >> 4) << 14); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt(vm_wait(N));
}

// vmcnt(n) for a value known after unrolling.
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 2: wait_vm<2>(); break;
    case 4: wait_vm<4>(); break;
    case 6: wait_vm<6>(); break;
    case 8: wait_vm<8>(); break;
    case 10: wait_vm<10>(); break;
    case 12: wait_vm<12>(); break;
    case 14: wait_vm<14>(); break;
    default: wait_vm<16>(); break;
  }
}

__device__ __forceinline__ void barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// (r, z) <- merge of two partial log-sum-exp states in base 2.
__device__ inline void lse_merge(float &r, float &z, float r2, float z2) {
  const float m = fmaxf(r, r2);
  if (m == -INFINITY) return;
  const float a = (r == -INFINITY) ? 0.0f : z * fast_exp2(r - m);
  const float b = (r2 == -INFINITY) ? 0.0f : z2 * fast_exp2(r2 - m);
  r = m;
  z = a + b;
}

// x + (the same register of lane l ^ 32): the same bits in both lanes.
__device__ inline float sum_halves(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Sum and maximum over the 32 lanes of a half-wave (l % 32), with the same
// bits in all of them: partners within quads (DPP quad permutations), then
// mirrored lanes of each 8 and of each 16 (DPP row mirrors), then the two
// 16-lane rows (permlane16 swap).  Every step combines two lanes' values
// with a commutative operation, so both partners hold the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <- 15 - i within 16
__device__ inline float other_row16(float x, float &mine) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  mine = __uint_as_float(sw[0]);
  return __uint_as_float(sw[1]);
}
__device__ inline float sum32(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  float a;
  const float b = other_row16(x, a);
  return a + b;
}
__device__ inline float max32(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  float a;
  const float b = other_row16(x, a);
  return fmaxf(a, b);
}

__device__ inline uint64_t ld_agent(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_agent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Which of a lane's rows see a key.  Rows see every key up to
// minlim = L - w (causal) or L - 1; past that, window row r sees keys up to
// L - w + r and the decode row sees all.  With rows numbered r * G + g, row
// x sees key k > L - w exactly when x >= (k - (L - w)) * G.  For the lane's
// rows base + c (c = out_row's offset), row base + c sees the key iff
// c >= the returned threshold; keys at or past kend (or before 0) are seen
// by none.
__device__ inline int vis_thr(int key, int kend, int minlim, int Lw, int G, int base) {
  if (key < 0 || key >= kend) return INT_MAX;
  if (key <= minlim) return INT_MIN;
  return (key - Lw) * G - base;
}

// Offset of this lane's i-th output row from its first (4 l / 32 + 32 tile).
__device__ __forceinline__ constexpr int row_off(int i) { return 8 * (i >> 2) + (i & 3); }

// Exclusive prefix sum over the workgroup; also returns the total.
__device__ __forceinline__ int block_exscan(int v, int *tmp, int &total) {
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

// Issues this wave's share of the block's 8 key tiles and of the halo tile
// into LDS: 16-byte position P = 128 wave + 64 u + lane of a tile receives
// chunk (P & 15) ^ (key & 15) of key row P >> 4, which leaves the tile
// swizzled (chunk c of key r at position c ^ (r & 15)), so the operand reads
// below are free of bank conflicts.  Keys past the block's end re-read its
// last key and halo keys outside the sequence are clamped into it, so every
// load is in bounds; such keys are masked or never used.  Exactly 18 loads
// per wave, two per tile, in tile order (the halo tile last).
__device__ inline void issue_block(const uint16_t *Kh, int64_t key0, int rowstride, int kb0, int kb1, int L,
                                   int wave, int lane) {
  typedef __attribute__((address_space(3))) void lds_void;
  typedef __attribute__((address_space(1))) void glb_void;
#pragma unroll
  for (int t = 0; t <= NTILE; ++t) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int P = 128 * wave + 64 * u + lane;
      const int row = P >> 4;
      const int csrc = (P & 15) ^ (row & 15);
      int key;
      if (t < NTILE) {
        key = min(kb0 + t * KT + row, kb1 - 1);
      } else {
        key = (row < HALO) ? kb0 - HALO + row : kb1 + (row - HALO);
        key = min(max(key, 0), L - 1);
      }
      const uint16_t *src = Kh + (key0 + key) * (int64_t)rowstride + csrc * 8;
      __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)(tile_at(t) + (128 * wave + 64 * u) * 16), 16, 0, 0);
    }
  }
}

// The 32 x 32 logits of this wave's row tile against key tile tl: the
// key fragments are read KSTEP k-steps at a time, to keep registers free.
constexpr int KSTEP = 2;
__device__ __forceinline__ f32x16 logits(const bf16x8 (&qf)[8], const char *tl, int lr, int hf) {
  f32x16 acc = {};
#pragma unroll
  for (int j0 = 0; j0 < 8; j0 += KSTEP) {
    bf16x8 kf[KSTEP];
#pragma unroll
    for (int j = 0; j < KSTEP; ++j)
      kf[j] = as_frag(*reinterpret_cast<const uint4 *>(tl + lr * ROWB + (((2 * (j0 + j) + hf) ^ (lr & 15)) << 4)));
#pragma unroll
    for (int j = 0; j < KSTEP; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[j0 + j], kf[j], acc, 0, 0, 0);
  }
  return acc;
}

// Row of this lane's i-th output entry within its row tile.
__device__ __forceinline__ int out_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }

__global__ __launch_bounds__(NT, 2) void resident_kernel(ResidentParams p, SegTable t) {
  __shared__ __attribute__((aligned(16))) float red[NW * SIDX];  // pass 2: per-row-tile key sums; merge scratch
  __shared__ __attribute__((aligned(16))) float sbuf[SIDX];      // S by position: [HALO + x], x in [-HALO, n + HALO)
  __shared__ float bias_s[kResMaxRows];
  __shared__ int tmp[NW];
  __shared__ int s_misc[4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;  // key of a tile
  const int hf = lane >> 5;  // chunk parity, and output rows 4 hf + ...
  const int rt = wave;       // row tile

  // ---- this call's token (used only once pass 1 is done; set by the kernel
  // that ran after the previous scoring launch, so a plain, scalar load),
  // and the block
  const uint64_t T = p.sync[0];
  const uint64_t tok = T + 1;
  int rem = blockIdx.x;
  int sb = 0, nb = 1;
  for (; sb < t.nseq; ++sb) {
    const int Ls = (int)(t.key_off[sb + 1] - t.key_off[sb]);
    nb = (Ls + BLK - 1) / BLK;
    if (rem < p.Hkv * nb) break;
    rem -= p.Hkv * nb;
  }
  if (sb >= t.nseq) return;  // more workgroups than blocks: never launched that way
  const int h = rem / nb;
  const int blk = rem - h * nb;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  const int segl = sb * p.Hkv + h;
  const int seg = t.seg0 + segl;
  const int b = t.seq0 + sb;
  const int kb0 = blk * BLK;
  const int kb1 = min(L, kb0 + BLK);
  const int n = kb1 - kb0;
  const int rowstride = p.Hkv * kHeadDim;
  const uint16_t *Kh = p.K + (int64_t)h * kHeadDim;
  const int nrt = p.Rp >> 5;     // row tiles of 32
  const bool active = rt < nrt;  // this wave owns rows (wave-uniform)

  // ---- query fragments of this wave's rows (loaded again wherever they are
  // needed after the key tiles' logits, so they hold no registers across the
  // waits).  Rows past R load row R - 1 instead: their statistics are never
  // used and their weight in pass 2 is 0.
  const uint16_t *qsrc;
  {
    const int row = min(rt * 32 + lr, p.R - 1);
    const int r = row / p.G;
    const int gi = row - r * p.G;
    qsrc = p.Q + ((int64_t)(b * p.wp + r) * p.Hq + h * p.G + gi) * (int64_t)kHeadDim + hf * 8;
  }
  auto load_q = [&](bf16x8 (&qf)[8]) {
    const uint16_t *src = qsrc;
    asm volatile("" : "+v"(src));  // a fresh load each time, not registers held from the last
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
#pragma unroll
    for (int j = 0; j < 8; ++j) qf[j] = __builtin_bit_cast(bf16x8, *(g_u32x4 *)(src + 16 * j));
  };
  const float cl2 = p.cl2;
  const int minlim = p.causal ? (L - p.w) : (L - 1);  // keys up to here are visible to every row
  const int Lw = L - p.w;
  const int rbase = rt * 32 + 4 * hf;  // this lane's first row

  uint64_t *flags = p.sync + kSyncFlags + 3 * p.nseg + (int64_t)segl * p.nblk_max;
  uint64_t *bflag = p.sync + kSyncFlags + p.nseg + seg;       // the segment's biases are published
  uint64_t *bclean = p.sync + kSyncFlags + 2 * p.nseg + seg;  // ... by a merger that saw every block
  uint32_t *hist_seg = p.seg_hist + (int64_t)seg * NBIN;
  float *lse_seg = p.lse + (int64_t)seg * p.nblk_max * p.Rp;
  float *bias_seg = p.biasg + (int64_t)seg * p.Rp;
  float *ref_seg = p.refg + (int64_t)seg * p.nblk_max * p.Rp;
  const bool merger = blk == 0;

  bf16x8 qf[8];
  load_q(qf);  // issued before the key tiles: every wait for a tile covers it
  issue_block(Kh, key0, rowstride, kb0, kb1, L, wave, lane);
  if (p.tables) {
    // this block's slice of the segment histogram, cleared before its flag
    const int z0 = (int)((int64_t)blk * NBIN / nb), z1 = (int)((int64_t)(blk + 1) * NBIN / nb);
    for (int i = z0 + tid; i < z1; i += NT) st_agent(hist_seg + i, 0u);
  }

  // Pass 1 (e for every (row, key) of the block, in registers), then the
  // row biases: block 0 of the segment merges every block's results once
  // they are all published and publishes the biases; the others wait for
  // them.  The loop body computes pass 1 for the block whose keys are in
  // LDS (cb): it runs again (same keys, same bits) after the block's sums
  // overflowed, with each row's true block maximum as its reference; after
  // a timed-out wait, for each block of the segment that has not published
  // (its keys loaded here, its results published for it by the same code,
  // so with the same bits it would publish itself); and at last for this
  // block again, whose e the waits' detour overwrote.
  const bool want_halo = p.pool_r > 0 && p.tables;
  float e[NTILE][16];
  float ref[16];
  int cb = blk;            // the block whose keys are in LDS
  bool true_max = false;   // ref holds each row's largest logit over block cb
  bool published = false;  // this block's results are out
  bool synced = false;     // waiting is over
  bool late = false;       // the segment histogram must not be added to
  int got = 0;             // 1 or 2: biases read from the merger (2: it saw some block late)
  bool missing = false;    // some block's results were computed here
  // The next block of the segment (from `from` on, ours excluded) that has
  // not published, or -1; the whole workgroup gets the same answer.
  auto next_missing = [&](int from) -> int {
    if (tid == 0) {
      int ob = from;
      while (ob < nb && (ob == blk || ld_agent(flags + ob) == tok)) ++ob;
      s_misc[3] = (ob < nb) ? ob : -1;
    }
    __syncthreads();
    const int r = s_misc[3];
    __syncthreads();
    return r;
  };
  // Keys of block c into LDS (after every wave is done with the last ones).
  auto load_block = [&](int c) {
    int c0 = c * BLK;
    asm volatile("" : "+s"(c0));  // addresses computed here, not held from the first issue
    __syncthreads();
    issue_block(Kh, key0, rowstride, c0, min(L, c0 + BLK), L, wave, lane);
    wait_vm<0>();
  };
#pragma unroll 1
  for (int round = 0;; ++round) {
    const int c0 = cb * BLK;
    const int c1 = min(L, c0 + BLK);
    const bool quick = (c1 - 1 <= minlim) && c1 - c0 == BLK;  // no key of the block is masked
    // The visibility thresholds are formed per tile, from a copy of the
    // block start that the compiler cannot see through: otherwise it
    // computes every tile's masks up front and holds them all.
    int kbr = c0;
    asm volatile("" : "+v"(kbr));
    if (round > 0) {
      load_q(qf);
      __syncthreads();  // every wave's key loads (waited for) have landed
    }
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
      if (round == 0) {
        // This wave's loads of tile tt have landed (tiles tt + 1 .. 8 may
        // still be in flight), then everyone's.
        wait_vm_upto(2 * (NTILE - tt));
        barrier();
      }
      // Every wave computes every tile, also a wave past the last row tile
      // (its rows repeat row R - 1) and a tile past the block's end (its
      // keys repeat the last one): the values are masked or never used, and
      // straight-line code keeps e in registers.
      const f32x16 acc = logits(qf, pair_at(tt >> 1) + (tt & 1) * TILE_BYTES, lr, hf);
      // acc[i]: row rt * 32 + out_row(i), key c0 + tt * 32 + lr.
      const int thr = vis_thr(kbr + tt * KT + lr, c1, minlim, Lw, p.G, rbase);
      if (tt == 0 && !true_max) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = acc[i] * cl2;
          if (!quick) x = (row_off(i) >= thr) ? x : -INFINITY;
          ref[i] = max32(x);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) e[tt][i] = fast_exp2(fmaf(acc[i], cl2, -ref[i]));
      if (!quick) {
#pragma unroll
        for (int i = 0; i < 16; ++i) e[tt][i] = (row_off(i) >= thr) ? e[tt][i] : 0.0f;
      }
    }
    // Each row's block sum; a sum past 2^100 (or not finite) anywhere in the
    // block is an overflow (rare): then every wave takes its rows' true
    // block maxima and the body runs again.
    float zr[16];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float z = e[0][i];
#pragma unroll
      for (int tt = 1; tt < NTILE; ++tt) z += e[tt][i];
      zr[i] = sum32(z);
      bad |= !(zr[i] <= kZLimit);
    }
    if (tid == 0) s_misc[0] = 0;
    __syncthreads();
    if (active && __ballot(bad) != 0ull && lane == 0) s_misc[0] = 1;
    __syncthreads();
    if (s_misc[0] && !true_max) {
      float m[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) m[i] = -INFINITY;
#pragma unroll 1
      for (int tt = 0; tt < NTILE; ++tt) {
        const f32x16 acc = logits(qf, tile_at(tt), lr, hf);
        const int thr = vis_thr(c0 + tt * KT + lr, c1, minlim, Lw, p.G, rbase);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (row_off(i) >= thr) m[i] = fmaxf(m[i], acc[i] * cl2);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ref[i] = max32(m[i]);
      true_max = true;
      continue;
    }

    if (cb != blk || !published) {
      // ---- publish log2 of each row's block sum (for block cb)
      if (active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float l2 = (zr[i] > 0.0f) ? ref[i] + __log2f(zr[i]) : -INFINITY;
          const int64_t at = (int64_t)cb * p.Rp + rt * 32 + out_row(i, hf);
          if (lr == 0) {
            st_agent(lse_seg + at, l2);
            st_agent(ref_seg + at, ref[i]);  // for the neighbours' halo keys
          }
        }
      }
      wait_vm<0>();  // this thread's stores are done
      __syncthreads();
      if (cb == blk) {
        if (tid == 0) {
          st_agent(flags + blk, tok);
          if (blockIdx.x == 0) st_agent(p.sync + 1, T);
        }
        published = true;
      }
    }
    if (cb != blk) {
      // on to the next block that has not published, else back to ours
      const int ob = next_missing(cb + 1);
      cb = (ob >= 0) ? ob : blk;
      true_max = false;
      load_block(cb);
      continue;
    }
    if (synced) break;

    // ---- wait: a non-merger for the merger's biases
    if (!merger) {
      if (wave == 0) {
        int it = 0, ok = 0;
        for (;;) {
          if (ld_agent(bflag) == tok) {
            ok = (ld_agent(bclean) == tok) ? 1 : 2;
            break;
          }
          if (++it > p.spin_cap) break;
          __builtin_amdgcn_s_sleep(2);
        }
        if (lane == 0) s_misc[1] = ok;
      }
      __syncthreads();
      got = s_misc[1];
      if (got) {
        late = got == 2;
        if (tid < p.Rp) bias_s[tid] = ld_agent(bias_seg + tid);
        __syncthreads();
        synced = true;
        break;
      }
      late = true;  // merging on its own: the histogram is not ours to add to
    }
    // ---- wait for every block's flag; past the bound, compute the blocks
    // that have not published here
    if (wave == 0) {
      int it = 0, give_up = 0;
      for (;;) {
        bool all = true;
        for (int b0 = 0; b0 < nb; b0 += 64) {
          const int bb = b0 + lane;
          const bool okb = bb >= nb || ld_agent(flags + bb) == tok;
          all = all && (__ballot(!okb) == 0ull);
        }
        if (all) break;
        if (++it > p.spin_cap) {
          give_up = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (lane == 0) s_misc[2] = give_up;
    }
    __syncthreads();
    synced = true;
    if (s_misc[2] == 0) break;
    late = true;
    const int ob = next_missing(0);
    if (ob < 0) break;  // every block published after all
    missing = true;
    cb = ob;
    true_max = false;
    load_block(cb);
  }

  if (got == 0) {
    // ---- merge: per row, log2 of the sum over the segment's blocks (the
    // largest value, then the sum of 2^(value - largest), in block order per
    // thread; the threads' partial results in thread order), minus log2 of
    // the row's weight.  Two rows per 8-byte device-scope load.
    const int npair = p.Rp >> 1;
    const int tpr = NT / npair;  // >= 4
    const int q = tid / tpr;
    const int sub = tid - q * tpr;
    float m0 = -INFINITY, s0 = 0.0f, m1 = -INFINITY, s1 = 0.0f;
    if (q < npair) {
      const uint64_t *src = reinterpret_cast<const uint64_t *>(lse_seg) + q;
      constexpr int MB = 16;  // loads in flight per thread
#pragma unroll 1
      for (int b0 = sub; b0 < nb; b0 += MB * tpr) {
        float v0[MB], v1[MB];
#pragma unroll
        for (int u = 0; u < MB; ++u) {
          const int bb = b0 + u * tpr;
          const uint64_t w = (bb < nb) ? ld_agent(src + (int64_t)bb * npair) : 0xff800000ff800000ull;  // -inf, -inf
          v0[u] = __uint_as_float((uint32_t)w);
          v1[u] = __uint_as_float((uint32_t)(w >> 32));
        }
        float a0 = v0[0], a1 = v1[0];
#pragma unroll
        for (int u = 1; u < MB; ++u) {
          a0 = fmaxf(a0, v0[u]);
          a1 = fmaxf(a1, v1[u]);
        }
        float t0 = 0.0f, t1 = 0.0f;
        if (a0 > -INFINITY) {
#pragma unroll
          for (int u = 0; u < MB; ++u) t0 += fast_exp2(v0[u] - a0);
        }
        if (a1 > -INFINITY) {
#pragma unroll
          for (int u = 0; u < MB; ++u) t1 += fast_exp2(v1[u] - a1);
        }
        lse_merge(m0, s0, a0, t0);
        lse_merge(m1, s1, a1, t1);
      }
    }
    float4 *part = reinterpret_cast<float4 *>(red);
    if (q < npair) part[q * tpr + sub] = make_float4(m0, s0, m1, s1);
    __syncthreads();
    if (q < npair && sub == 0) {
      for (int k = 1; k < tpr; ++k) {
        const float4 o = part[q * tpr + k];
        lse_merge(m0, s0, o.x, o.y);
        lse_merge(m1, s1, o.z, o.w);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int row = 2 * q + h2;
        const float m = h2 ? m1 : m0, sm = h2 ? s1 : s0;
        const int wr = row / p.G;  // window rows 0 .. w-1, then the decode row
        float lc;                  // log2 of the row's weight c_r
        if (p.weighting == 1) {
          lc = p.lam2 * (float)(wr - (p.w - 1) - p.has_decode) - p.log2norm;
        } else {
          float c = 1.0f;
          if (p.has_decode) c = (wr < p.w) ? (1.0f - p.alpha) : p.alpha;
          lc = (c > 0.0f) ? __log2f(c) : -INFINITY;
        }
        float out = INFINITY;  // a row of weight 0 contributes nothing
        if (row < p.R && lc > -INFINITY && sm > 0.0f) out = m + __log2f(sm) - lc;
        bias_s[row] = out;
      }
    }
    __syncthreads();
    if (merger) {
      if (tid < p.Rp) st_agent(bias_seg + tid, bias_s[tid]);
      wait_vm<0>();
      __syncthreads();
      if (tid == 0) {
        if (!missing) st_agent(bclean, tok);
        wait_vm<0>();
        st_agent(bflag, tok);
      }
    }
  }
  if (tid == 0 && p.tables && late) st_agent(p.sync + kSyncFlags + seg, tok);  // the histogram is incomplete

  // ---- pass 2: S per key from the stored e; the halo tile's logits afresh
  // (its keys are still in LDS; the query fragments are loaded again, which
  // kept them out of registers while e was held)
  if (active) {
    // the halo's loads first, so that they land while the block's sums run
    const int hpos = (lr < HALO) ? kb0 - HALO + lr : kb1 + lr - HALO;
    const int hthr = vis_thr(hpos, L, minlim, Lw, p.G, rbase);
    float href[16];  // reference logits of the block that holds the halo key
    if (want_halo) {
      load_q(qf);
      const int ob = (lr < HALO) ? blk - 1 : blk + 1;  // the block that holds hpos, if hpos is in the sequence
      const float *oref = ref_seg + (int64_t)min(max(ob, 0), nb - 1) * p.Rp + rt * 32;
#pragma unroll
      for (int i = 0; i < 16; ++i) href[i] = (hthr == INT_MAX) ? 0.0f : ld_agent(oref + out_row(i, hf));
    }
    float f[16];  // 2^(ref - bias): e times f is the row's weighted probability
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = fast_exp2(ref[i] - bias_s[rt * 32 + out_row(i, hf)]);
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
      float s = e[tt][0] * f[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) s = fmaf(e[tt][i], f[i], s);
      s = sum_halves(s);
      if (hf == 0) red[rt * SIDX + tt * KT + lr] = s;
    }
    if (want_halo) {
      // The halo keys' S exactly as the blocks they belong to compute it:
      // with that block's reference logits (published with its sums), the
      // same masking, products and order of summation.
      const f32x16 acc = logits(qf, g_halo, lr, hf);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float ev = (row_off(i) >= hthr) ? fast_exp2(fmaf(acc[i], cl2, -href[i])) : 0.0f;
        const float fv = fast_exp2(href[i] - bias_s[rt * 32 + out_row(i, hf)]);
        s = (i == 0) ? ev * fv : fmaf(ev, fv, s);
      }
      s = sum_halves(s);
      if (hf == 0) red[rt * SIDX + BLK + lr] = s;
    }
  }
  __syncthreads();

  // ---- S by position (the sum over the row tiles in order)
  const bool is_max = p.pool == 2;
  const float fill = is_max ? -INFINITY : 0.0f;  // the pool's value outside the sequence
  const int64_t segbase = (int64_t)p.Hkv * key0 + (int64_t)h * L;
  {
    const int nx = (p.pool_r > 0 && p.tables) ? SIDX : BLK;
    for (int x = tid; x < nx; x += NT) {
      int pos;
      if (x < BLK) {
        if (x >= n) continue;
        pos = kb0 + x;
      } else if (x < BLK + HALO) {
        pos = kb0 - HALO + (x - BLK);
      } else {
        pos = kb1 + (x - BLK - HALO);
      }
      float v = 0.0f;
      for (int r2 = 0; r2 < nrt; ++r2) v += red[r2 * SIDX + x];
      if (x < BLK && p.scores) p.scores[segbase + pos] = v;
      if (pos < 0 || pos >= L) v = fill;
      sbuf[HALO + pos - kb0] = v;
    }
  }
  if (!p.tables) return;
  __syncthreads();

  // ---- pool, pooled output
  const int x = tid;
  float P = 0.0f;
  if (x < n) {
    const float *c = sbuf + HALO + x;
    const int r = p.pool_r;
    if (r == 0) {
      P = c[0];
    } else if (is_max) {
      float m = c[0];
      for (int j = -r; j <= r; ++j) m = fmaxf(m, c[j]);
      P = m;
    } else {
      float sum = 0.0f;
      for (int j = -r; j <= r; ++j) sum += c[j];
      P = sum / p.pool_width;
    }
    p.pooled[segbase + kb0 + x] = P;
  }

  // ---- counting sort of the block by first digit; the segment histogram
  // (the key tiles are no longer needed: the histogram lives in their LDS)
  uint32_t *hist = reinterpret_cast<uint32_t *>(g_pair0);
  reinterpret_cast<uint4 *>(hist)[2 * tid] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4 *>(hist)[2 * tid + 1] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  uint32_t key = 0u, dg = 0u, rank = 0u;
  if (x < n) {
    key = select_key(P, kb0 + x, L, p.sink, p.recent);
    const int64_t rel = ((int64_t)key - (int64_t)order_key(p.wsum / (float)L)) >> DSHIFT;
    dg = (uint32_t)min<int64_t>(NBIN - 1, max<int64_t>(0, rel + NBIN / 2));
    rank = atomicAdd(&hist[dg], 1u);
  }
  __syncthreads();
  uint32_t cnt[8], pre[8];
  {
    const uint4 a0 = reinterpret_cast<const uint4 *>(hist)[2 * tid];
    const uint4 a1 = reinterpret_cast<const uint4 *>(hist)[2 * tid + 1];
    cnt[0] = a0.x; cnt[1] = a0.y; cnt[2] = a0.z; cnt[3] = a0.w;
    cnt[4] = a1.x; cnt[5] = a1.y; cnt[6] = a1.z; cnt[7] = a1.w;
  }
  int own = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) own += (int)cnt[u];
  int total;
  uint32_t run = (uint32_t)block_exscan(own, tmp, total);  // its barriers end the reads above
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    pre[u] = run;
    run += cnt[u];
  }
  const int64_t tabi = (int64_t)seg * p.nblk_max + blk;
  reinterpret_cast<uint4 *>(p.tab + tabi * NBIN)[tid] =
      make_uint4(pre[0] | (pre[1] << 16), pre[2] | (pre[3] << 16), pre[4] | (pre[5] << 16), pre[6] | (pre[7] << 16));
  if (!late) {  // a block that did not see every block publish marked the histogram incomplete instead
    uint32_t *sh = hist_seg + 8 * tid;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (cnt[u]) atomicAdd(sh + u, cnt[u]);
  }
  reinterpret_cast<uint4 *>(hist)[2 * tid] = make_uint4(pre[0], pre[1], pre[2], pre[3]);
  reinterpret_cast<uint4 *>(hist)[2 * tid + 1] = make_uint4(pre[4], pre[5], pre[6], pre[7]);
  __syncthreads();
  if (x < n) p.bucket[tabi * BLK + hist[dg] + rank] = key;
}

__global__ void bump_kernel(uint64_t *sync) {
  if (threadIdx.x == 0) sync[0] = sync[1] + 1;
}

}  // namespace

// The next call's token, after a scoring launch that has no selection
// behind it (the selection kernel sets it otherwise).
hipError_t launch_resident_bump(uint64_t *sync, hipStream_t s) {
  hipLaunchKernelGGL(bump_kernel, dim3(1), dim3(64), 0, s, sync);
  return hipGetLastError();
}

hipError_t launch_resident(const ResidentParams &p, const SegTable &t, int items, hipStream_t s) {
  if (items < 1) return hipSuccess;
  hipLaunchKernelGGL(resident_kernel, dim3(items), dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel
