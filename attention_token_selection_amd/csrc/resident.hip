// Resident scoring: TideKV's two-pass blockwise procedure ("Delayed KV
// Eviction via Layer-Wise Chunked Prefill", §4.2) with each key block read
// from memory once.
//
// Work unit: one workgroup of eight waves per block of 512 keys of one
// (sequence, KV head) segment.  The block's keys (128 KiB) are loaded
// straight from memory into LDS (global_load_lds, 16 bytes per lane, every
// tile's loads issued up front) and stay there for both passes:
//
//  1. pass 1: the logits of the block against the segment's observation rows
//     and, per row, log2 of the block's sum of exponentials (online, with a
//     lazily raised reference);
//  2. the per-row results are published, and the workgroup waits until every
//     block of its segment has published, then merges them in block order
//     into each row's normaliser;
//  3. pass 2 over the same LDS-resident keys, plus a halo tile (the 16 keys
//     before and after the block, for the pool): c_r * p_r summed over the
//     rows of the group (TideKV §4.2 aggregation; DeferKV guide, Phase 2 row
//     weights);
//  4. the 1-D pool of the block's positions, the pooled scores written out,
//     and the block's counting sort by a first digit of each pooled value's
//     order key: the exclusive prefix of the block's digit histogram, the
//     keys grouped by digit, and the histogram added to the segment's.  The
//     selection kernel finishes the top-k from these.
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
// needs clearing), and polls its segment's flags.  The wait is bounded:
// after spin_cap polls the block computes pass 1 of the blocks that have
// not published yet itself (the same code on the same keys, so the same
// bits) and goes on, so the kernel ends whatever else shares the GPU and in
// whatever order its workgroups run.  Such a block leaves the segment's
// histogram alone and marks it incomplete; the selection then rebuilds it
// from the blocks' tables.  Before publishing, every block clears its slice
// of the segment histogram, so the histogram is clear before any block
// that saw all flags adds to it.  Cross-workgroup data moves with
// device-scope atomic loads and stores (coherent across the chip's L2s
// without cache write-backs); a block's results are complete before its
// flag is set.
//
// Rows and keys: the R = G * w' observation rows of the KV head (row =
// window row * G + query head of the group) are split into row tiles of 32.
// With at most four row tiles, waves 0-3 own row tiles 0-3 over the even
// key tiles of the block and waves 4-7 the same rows over the odd ones
// (two key groups, so that each key tile is read from LDS by four waves,
// not eight); with five to eight, wave v owns row tile v over every key
// tile.  Contraction: v_mfma_f32_32x32x16_bf16 over d = 128 in 8 k-steps;
// lane l supplies, at k-step j, the 16-byte chunk 2 j + l / 32 of entry
// l % 32 of each operand (the same permutation of the contraction index on
// both operands leaves the products unchanged).  Pass 1 puts keys in the
// first operand (a lane holds 16 keys of one row), pass 2 rows (a lane
// holds 16 rows of one key).
#include <algorithm>

#include "kvsel_internal.h"
#include "kvsel_device.h"

namespace kvsel {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NT = kResThreads;        // 512 threads
constexpr int NW = NT / 64;            // 8 waves
constexpr int KT = kKeyTile;           // 32 keys per tile
constexpr int BLK = kResBlock;         // 512 keys per workgroup
constexpr int NTILE = BLK / KT;        // 16 tiles
constexpr int ROWB = kHeadDim * 2;     // 256 bytes per key row
constexpr int TILE_BYTES = KT * ROWB;  // 8 KiB
constexpr int HALO = kResHalo;         // 16
constexpr int SIDX = BLK + 2 * HALO;   // per-wave key sums: block keys, then the halo tile's
constexpr int NBIN = kResBins;         // 2048
constexpr int DSHIFT = kResDigitShift; // 21
constexpr float kZLimit = 0x1p100f;    // a lane's running sum stays below this
static_assert(TILE_BYTES == NT * 16, "one 16-byte chunk per lane and tile");
static_assert(NT == BLK, "one thread per position of a block in the epilogue");
static_assert(NBIN == 4 * NT, "four bins per thread in the block scan");
static_assert(NBIN == 2048, "digits centre on bin 1024");
static_assert(kResMaxRows == NW * 32, "one row tile of 32 per wave");

// The block's key tiles in LDS, two per array: an unrolled step names its
// pair's array, so the compiler waits only for that pair's loads (an array
// it cannot tell apart from the others would make it wait for all of them).
#define KVSEL_PAIR(n) __shared__ __attribute__((aligned(16))) char g_pair##n[2 * TILE_BYTES];
KVSEL_PAIR(0) KVSEL_PAIR(1) KVSEL_PAIR(2) KVSEL_PAIR(3) KVSEL_PAIR(4) KVSEL_PAIR(5) KVSEL_PAIR(6) KVSEL_PAIR(7)
#undef KVSEL_PAIR
__shared__ __attribute__((aligned(16))) char g_halo[TILE_BYTES];

__device__ __forceinline__ char *pair_at(int i) {
  switch (i) {
    case 0: return g_pair0;
    case 1: return g_pair1;
    case 2: return g_pair2;
    case 3: return g_pair3;
    case 4: return g_pair4;
    case 5: return g_pair5;
    case 6: return g_pair6;
    default: return g_pair7;
  }
}

// Key tile t (0 .. 15), or the halo tile (t = 16).
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
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    case 8: wait_vm<8>(); break;
    case 9: wait_vm<9>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    case 12: wait_vm<12>(); break;
    case 13: wait_vm<13>(); break;
    case 14: wait_vm<14>(); break;
    case 15: wait_vm<15>(); break;
    default: wait_vm<16>(); break;
  }
}

__device__ __forceinline__ void barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// (r, z) <- merge of two partial log-sum-exp states in base 2.  Symmetric in
// its operands bit for bit, so exchange partners agree exactly.
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

__device__ inline uint64_t ld_agent(const uint64_t *p) {
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

// Observation row -> last key it sees.
__device__ inline int row_limit(int row, const ResidentParams &p, int L) {
  const int r = row / p.G;
  if (!p.causal || r >= p.w) return L - 1;
  return L - p.w + r;
}

// Exclusive prefix sum over the 512 threads; also returns the total.
__device__ __forceinline__ int block_exscan512(int v, int *tmp, int &total) {
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

// Issues this wave's share of the block's 16 key tiles and of the halo tile
// into LDS: 16-byte position P = 64 wave + lane of a tile receives chunk
// (P & 15) ^ (key & 15) of key row P >> 4, which leaves the tile swizzled
// (chunk c of key r at position c ^ (r & 15)), so the operand reads below
// are free of bank conflicts.  Keys past the block's end re-read its last
// key and halo keys outside the sequence are clamped into it, so every load
// is in bounds; such keys are masked or never used.  Exactly 17 loads per
// wave, in tile order.
__device__ inline void issue_block(const uint16_t *Kh, int64_t key0, int rowstride, int kb0, int kb1, int L,
                                   int wave, int lane) {
  const int P = 64 * wave + lane;
  const int row = P >> 4;
  const int csrc = (P & 15) ^ (row & 15);
  const uint16_t *base = Kh + key0 * (int64_t)rowstride + csrc * 8;
  typedef __attribute__((address_space(3))) void lds_void;
  typedef __attribute__((address_space(1))) void glb_void;
#pragma unroll
  for (int t = 0; t < NTILE; ++t) {
    const int key = min(kb0 + t * KT + row, kb1 - 1);
    __builtin_amdgcn_global_load_lds((glb_void *)(base + (int64_t)key * rowstride),
                                     (lds_void *)(tile_at(t) + wave * 1024), 16, 0, 0);
  }
  int hk = (row < HALO) ? kb0 - HALO + row : kb1 + (row - HALO);
  hk = min(max(hk, 0), L - 1);
  __builtin_amdgcn_global_load_lds((glb_void *)(base + (int64_t)hk * rowstride),
                                   (lds_void *)(g_halo + wave * 1024), 16, 0, 0);
}

// This lane's operand fragments of a tile (8 k-steps): entry l % 32, chunk
// 2 j + l / 32, swizzled.
__device__ __forceinline__ void read_tile(bf16x8 (&kf)[8], const char *tl, int lr, int hf) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    kf[j] = as_frag(*reinterpret_cast<const uint4 *>(tl + lr * ROWB + (((2 * j + hf) ^ (lr & 15)) << 4)));
}

// KG: key groups (2: up to four row tiles, the two groups taking alternate
// key tiles; 1: five to eight row tiles, each wave every key tile).
template <int KG>
__global__ __launch_bounds__(NT) void resident_kernel(ResidentParams p, SegTable t) {
  constexpr int NRTW = NW / KG;  // row tiles one key group covers
  __shared__ __attribute__((aligned(16))) float red[NW * SIDX];  // pass 2: per-row-tile key sums; also scratch
  __shared__ __attribute__((aligned(16))) float sbuf[SIDX];      // S by position: [HALO + x], x in [-HALO, n + HALO)
  __shared__ float bias_s[kResMaxRows];
  __shared__ float2 xch[kResMaxRows];                             // pass 1: the odd key group's row states
  __shared__ int tmp[NW];
  __shared__ int s_misc[4];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 31;  // entry of a 32-wide operand
  const int hf = lane >> 5;  // chunk parity, and output rows 4 hf + ...
  const int rt = wave % NRTW;
  const int kg = wave / NRTW;

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
  const int nrt = p.Rp >> 5;        // row tiles of 32
  const bool active = rt < nrt;     // this wave owns rows (wave-uniform)

  // ---- query fragments of this wave's rows, issued before the key tiles so
  // that every wait for a tile below also covers them.  Rows past R load
  // row R - 1 instead (no branch, so nothing waits for these loads before
  // the tiles are issued): their statistics are never used and their
  // weight in pass 2 is 0.
  bf16x8 qf[8];
  {
    const int row = min(rt * 32 + lr, p.R - 1);
    const int r = row / p.G;
    const int gi = row - r * p.G;
    const uint16_t *src = p.Q + ((int64_t)(b * p.wp + r) * p.Hq + h * p.G + gi) * (int64_t)kHeadDim + hf * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) qf[j] = as_frag(*reinterpret_cast<const uint4 *>(src + 16 * j));
  }

  const float cl2 = p.cl2;
  const int minlim = p.causal ? (L - p.w) : (L - 1);  // keys up to here are visible to every row
  const int lim1 = row_limit(rt * 32 + lr, p, L);
  float *lse_seg = p.lse + (int64_t)seg * p.nblk_max * p.Rp;

  // Pass 1 of block ob (keys c0 .. c1 - 1): loads it into LDS, then log2 of
  // each row's sum of exponentials over the block, published to lse.
  //
  // Pairs of tiles whose keys every row sees run first, in an unrolled loop
  // that waits for each pair's own loads: a wave's first tile gives each
  // lane its reference (its largest logit there), later tiles only add.
  // The other tiles (past the block's end, or inside the window's causal
  // triangle) run once every load has landed, with masks and a reference
  // raised whenever the running sum would pass 2^100.  A wave whose quick
  // sums passed that bound redoes the whole block the careful way.
  auto pass1 = [&](int ob, int c0, int c1) {
    issue_block(Kh, key0, rowstride, c0, c1, L, wave, lane);
    const int nc = c1 - c0;
    const int nvis = (min(c1 - 1, minlim) - c0 + 1) / KT;  // leading tiles all rows see in full
    const int nfp = max(0, min(nvis, NTILE)) >> 1;          // ... as pairs
    float ref = -INFINITY, zs = 0.0f;
#pragma unroll
    for (int tp = 0; tp < NTILE; tp += 2) {
      if ((tp >> 1) < nfp) {
        // This wave's parts of tiles tp and tp + 1 have landed (17 loads in
        // tile order: tiles tp + 2 .. 16 may still be in flight), then everyone's.
        wait_vm_upto(NTILE - (tp + 1));
        barrier();
        if (active) {
#pragma unroll
          for (int u = 0; u < 2 / KG; ++u) {
            bf16x8 kf[8];
            read_tile(kf, pair_at(tp >> 1) + ((KG == 2) ? kg : u) * TILE_BYTES, lr, hf);
            f32x16 acc = {};
#pragma unroll
            for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[j], acc, 0, 0, 0);
            // acc[i]: key 8 (i / 4) + 4 hf + i % 4 of the tile, row rt * 32 + lr.
            if (tp == 0 && u == 0) {
              float m = -INFINITY;
#pragma unroll
              for (int i = 0; i < 16; ++i) m = fmaxf(m, acc[i] * cl2);
              ref = m;
            }
            float e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) e[i] = fast_exp2(fmaf(acc[i], cl2, -ref));
            const float a = ((e[0] + e[8]) + (e[4] + e[12])) + ((e[1] + e[9]) + (e[5] + e[13]));
            const float c = ((e[2] + e[10]) + (e[6] + e[14])) + ((e[3] + e[11]) + (e[7] + e[15]));
            zs += a + c;
          }
        }
      }
    }
    wait_vm<0>();
    barrier();
    // The rest, and a redo by a wave whose quick sums went past the bound.
    int g0 = 2 * nfp;
    if (__ballot(active && !(zs <= kZLimit)) != 0ull) {
      g0 = 0;
      ref = -INFINITY;
      zs = 0.0f;
    }
    const int ntl = (nc + KT - 1) / KT;
    if (active) {
      for (int tt = g0 + ((KG == 2) ? kg : 0); tt < ntl; tt += KG) {
        bf16x8 kf[8];
        read_tile(kf, tile_at(tt), lr, hf);
        f32x16 acc = {};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[j], acc, 0, 0, 0);
        const int kbase = c0 + tt * KT;
        const bool need_mask = (kbase + KT - 1 > minlim) || (kbase + KT - 1 >= c1);
        float e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = fast_exp2(fmaf(acc[i], cl2, -ref));
          const int key = kbase + 8 * (i >> 2) + 4 * hf + (i & 3);
          e[i] = (need_mask && (key > lim1 || key >= c1)) ? 0.0f : v;
        }
        const float a = ((e[0] + e[8]) + (e[4] + e[12])) + ((e[1] + e[9]) + (e[5] + e[13]));
        const float c = ((e[2] + e[10]) + (e[6] + e[14])) + ((e[3] + e[11]) + (e[7] + e[15]));
        const float znew = zs + (a + c);
        if (__builtin_expect(__ballot(!(znew <= kZLimit)) != 0ull, 0)) {
          // Raise the reference to the largest visible logit seen so far and
          // redo this tile's sum (always on a careful pass's first tile).
          float m = ref;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (!need_mask || (key <= lim1 && key < c1)) m = fmaxf(m, acc[i] * cl2);
          }
          float z = (ref == -INFINITY || m == -INFINITY) ? 0.0f : zs * fast_exp2(ref - m);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (!need_mask || (key <= lim1 && key < c1)) z += fast_exp2(fmaf(acc[i], cl2, -m));
          }
          ref = m;
          zs = z;
        } else {
          zs = znew;
        }
      }
    }
    // The two lanes of a row hold different keys: merge them (the same bits
    // in both); then the key groups, in order; publish log2 of the row's
    // block sum.
    {
      float r2 = __shfl_xor(ref, 32), z2 = __shfl_xor(zs, 32);
      lse_merge(ref, zs, r2, z2);
    }
    const int row = rt * 32 + lr;
    if (KG == 2) {
      if (active && kg == 1 && hf == 0) xch[row] = make_float2(ref, zs);
      __syncthreads();
      if (active && kg == 0) lse_merge(ref, zs, xch[row].x, xch[row].y);
    }
    if (active && kg == 0 && hf == 0) {
      const float l2 = (zs > 0.0f) ? ref + __log2f(zs) : -INFINITY;
      st_agent(lse_seg + (int64_t)ob * p.Rp + row, l2);
    }
  };

  // ---- pass 1 of our block, publish, wait for the segment's other blocks.
  // After a wait that times out: pass 1 of every block of the segment that
  // has not published (its owner writes the same bits when it gets to it),
  // then our own keys again.
  uint64_t *flags = p.sync + kSyncIncomplete + p.nseg + (int64_t)segl * p.nblk_max;
  uint32_t *hist_seg = p.seg_hist + (int64_t)seg * NBIN;
  if (p.tables) {
    // this block's slice of the segment histogram, cleared before its flag
    const int z0 = (int)((int64_t)blk * NBIN / nb), z1 = (int)((int64_t)(blk + 1) * NBIN / nb);
    for (int i = z0 + tid; i < z1; i += NT) st_agent(hist_seg + i, 0u);
  }
  int ob = blk;
  int scan = 0;  // next block the late path looks at
  bool late = false;
  for (;;) {
    const int c0 = ob * BLK;
    pass1(ob, c0, min(L, c0 + BLK));
    wait_vm<0>();  // this thread's stores (and the halo tile) are done
    __syncthreads();
    if (!late) {
      if (tid == 0) {
        st_agent(flags + blk, tok);
        if (blockIdx.x == 0) st_agent(p.sync + 1, T);
      }
      if (wave == 0) {
        // poll the segment's flags, 64 per load, until all carry the token
        int it = 0;
        bool give_up = false;
        for (;;) {
          bool all = true;
          for (int b0 = 0; b0 < nb; b0 += 64) {
            const int bb = b0 + lane;
            const bool ok = bb >= nb || ld_agent(flags + bb) == tok;
            all = all && (__ballot(!ok) == 0ull);
          }
          if (all) break;
          if (++it > p.spin_cap) {
            give_up = true;
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
        if (lane == 0) s_misc[1] = give_up ? 1 : 0;
      }
      __syncthreads();
      late = s_misc[1] != 0;
      if (!late) break;
      if (tid == 0 && p.tables) st_agent(p.sync + kSyncIncomplete + seg, tok);
    }
    int next = -1;
    while (scan < nb) {
      const int cand = scan++;
      if (cand == blk) continue;
      if (tid == 0) s_misc[2] = (ld_agent(flags + cand) == tok) ? 1 : 0;
      __syncthreads();
      const int done = s_misc[2];
      __syncthreads();
      if (!done) {
        next = cand;
        break;
      }
    }
    if (next < 0) {
      issue_block(Kh, key0, rowstride, kb0, kb1, L, wave, lane);
      wait_vm<0>();
      __syncthreads();
      break;
    }
    ob = next;
  }

  // ---- merge: per row, log2 of the sum over the segment's blocks, minus
  // log2 of the row's weight.  The blocks' results are read with
  // device-scope loads (coherent across the chip's L2s), two rows per 8-byte
  // load; tpr threads share a row pair, each taking every tpr-th block: the
  // largest value, then the sum of 2^(value - largest), in block order;
  // then the threads' partial results in thread order (a fixed order, so
  // every block of the segment gets the same bits).
  {
    const int npair = p.Rp >> 1;
    const int tpr = NT / npair;  // >= 4
    const int q = tid / tpr;
    const int sub = tid - q * tpr;
    float m0 = -INFINITY, s0 = 0.0f, m1 = -INFINITY, s1 = 0.0f;
    if (q < npair) {
      const uint64_t *src = reinterpret_cast<const uint64_t *>(lse_seg) + q;
      for (int b0 = sub; b0 < nb; b0 += 16 * tpr) {
        float v0[16], v1[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int bb = b0 + u * tpr;
          const uint64_t w = (bb < nb) ? ld_agent(src + (int64_t)bb * npair) : 0xff800000ff800000ull;  // -inf, -inf
          v0[u] = __uint_as_float((uint32_t)w);
          v1[u] = __uint_as_float((uint32_t)(w >> 32));
        }
        float a0 = v0[0], a1 = v1[0];
#pragma unroll
        for (int u = 1; u < 16; ++u) {
          a0 = fmaxf(a0, v0[u]);
          a1 = fmaxf(a1, v1[u]);
        }
        float t0 = 0.0f, t1 = 0.0f;
        if (a0 > -INFINITY) {
#pragma unroll
          for (int u = 0; u < 16; ++u) t0 += fast_exp2(v0[u] - a0);
        }
        if (a1 > -INFINITY) {
#pragma unroll
          for (int u = 0; u < 16; ++u) t1 += fast_exp2(v1[u] - a1);
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
  }

  // ---- pass 2 over the resident keys (and the halo tile when pooling)
  {
    float bia[16];
    int lim2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = rt * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
      bia[i] = active ? bias_s[row] : INFINITY;
      lim2[i] = row_limit(row, p, L);
    }
    const int nbt = (n + KT - 1) / KT;  // block tiles in use
    const bool halo_on = p.pool_r > 0 && p.tables;
    // leading tiles that every row sees in full, as pairs: no masks
    const int nfp = max(0, min((min(kb1 - 1, minlim) - kb0 + 1) / KT, nbt)) >> 1;
    if (active) {
      for (int st = 0; st < nfp; ++st) {
#pragma unroll
        for (int u = 0; u < 2 / KG; ++u) {
          const int tt = 2 * st + ((KG == 2) ? kg : u);
          bf16x8 kf[8];
          read_tile(kf, pair_at(st) + (tt & 1) * TILE_BYTES, lr, hf);
          f32x16 acc = {};
#pragma unroll
          for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[j], kf[j], acc, 0, 0, 0);
          // acc[i]: row rt * 32 + 8 (i / 4) + 4 hf + i % 4, key tt * 32 + lr.
          float e[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) e[i] = fast_exp2(fmaf(acc[i], cl2, -bia[i]));
          const float a = ((e[0] + e[8]) + (e[4] + e[12])) + ((e[1] + e[9]) + (e[5] + e[13]));
          const float c = ((e[2] + e[10]) + (e[6] + e[14])) + ((e[3] + e[11]) + (e[7] + e[15]));
          const float sk = sum_halves(a + c);
          if (hf == 0) red[rt * SIDX + tt * KT + lr] = sk;
        }
      }
      // the remaining block tiles, then the halo tile (key group 0), with masks
      const int nend = nbt + (halo_on ? 1 : 0);
      for (int tt0 = 2 * nfp; tt0 < nend; ++tt0) {
        const bool halo = tt0 >= nbt;
        if (KG == 2 && (halo ? 0 : (tt0 & 1)) != kg) continue;
        bf16x8 kf[8];
        read_tile(kf, tile_at(halo ? NTILE : tt0), lr, hf);
        f32x16 acc = {};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[j], kf[j], acc, 0, 0, 0);
        const int pos = halo ? ((lr < HALO) ? kb0 - HALO + lr : kb1 + lr - HALO) : kb0 + tt0 * KT + lr;
        float e[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float v = fast_exp2(fmaf(acc[i], cl2, -bia[i]));
          e[i] = (pos > lim2[i]) ? 0.0f : v;
        }
        const float a = ((e[0] + e[8]) + (e[4] + e[12])) + ((e[1] + e[9]) + (e[5] + e[13]));
        const float c = ((e[2] + e[10]) + (e[6] + e[14])) + ((e[3] + e[11]) + (e[7] + e[15]));
        const float sk = sum_halves(a + c);
        if (hf == 0) red[rt * SIDX + (halo ? BLK : tt0 * KT) + lr] = sk;
      }
    }
  }
  __syncthreads();

  // ---- S by position (the sum over the waves' rows in wave order)
  const bool is_max = p.pool == 2;
  const float fill = is_max ? -INFINITY : 0.0f;  // the pool's value outside the sequence
  const int nwr = nrt;                            // row tiles with partial sums
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
      for (int w2 = 0; w2 < nwr; ++w2) v += red[w2 * SIDX + x];
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
  uint32_t *hist = reinterpret_cast<uint32_t *>(red);
  reinterpret_cast<uint4 *>(hist)[tid] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  uint32_t key = 0u, dg = 0u, rank = 0u;
  if (x < n) {
    key = select_key(P, kb0 + x, L, p.sink, p.recent);
    const int64_t rel = ((int64_t)key - (int64_t)order_key(p.wsum / (float)L)) >> DSHIFT;
    dg = (uint32_t)min<int64_t>(NBIN - 1, max<int64_t>(0, rel + NBIN / 2));
    rank = atomicAdd(&hist[dg], 1u);
  }
  __syncthreads();
  const uint4 c4 = reinterpret_cast<const uint4 *>(hist)[tid];
  int total;
  const int ex = block_exscan512((int)(c4.x + c4.y + c4.z + c4.w), tmp, total);  // its barriers end the reads above
  const uint32_t p0 = (uint32_t)ex, p1 = p0 + c4.x, p2 = p1 + c4.y, p3 = p2 + c4.z;
  const int64_t tabi = (int64_t)seg * p.nblk_max + blk;
  reinterpret_cast<uint2 *>(p.tab + tabi * NBIN)[tid] = make_uint2(p0 | (p1 << 16), p2 | (p3 << 16));
  if (!late) {  // a block that stopped waiting has marked the histogram incomplete instead
    uint32_t *sh = hist_seg + 4 * tid;
    if (c4.x) atomicAdd(sh, c4.x);
    if (c4.y) atomicAdd(sh + 1, c4.y);
    if (c4.z) atomicAdd(sh + 2, c4.z);
    if (c4.w) atomicAdd(sh + 3, c4.w);
  }
  reinterpret_cast<uint4 *>(hist)[tid] = make_uint4(p0, p1, p2, p3);
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
  if (p.Rp > 128)
    hipLaunchKernelGGL(resident_kernel<1>, dim3(items), dim3(NT), 0, s, p, t);
  else
    hipLaunchKernelGGL(resident_kernel<2>, dim3(items), dim3(NT), 0, s, p, t);
  return hipGetLastError();
}

}  // namespace kvsel
