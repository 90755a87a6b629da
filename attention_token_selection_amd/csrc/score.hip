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
// block's per-row state is stored; a small merge launch then combines the
// blocks, in a fixed order, into per row bias = r + log2(Z) - log2(c_r).
//
// Pass 2 puts the observation rows in M (A = Q, B = K), so each lane holds 16
// rows of one key: it adds c_r * p = 2^(x - bias) over its rows in-lane, the
// two lane halves are combined with one swap, the four waves in LDS, in a
// fixed order (no floating-point atomics: results are bit-reproducible).
#include "kvsel_internal.h"

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
constexpr int PD = 4;                    // LDS ring slots; tiles in flight = PD - 1
// s_waitcnt immediate for vmcnt(2 (PD - 2)) with the other counters left alone.
constexpr int kWaitTile = 0x3F70 | (2 * (PD - 2));
static_assert(PD == 4 && 2 * (PD - 2) < 16, "four named slots; vmcnt fits the low field");
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

// Issues this wave's share of key tile i0 .. i0+31 (`kt` = its first key row
// of this head) straight into the LDS slot: 16-byte position P = 128 * wave
// + 64 * i + lane (i = 0, 1) of the slot receives chunk (P & 15) ^ (row & 15)
// of key row = P >> 4, which leaves the slot in the swizzled layout.  Rows
// past `rmax` (the block's last key minus i0) re-read that key, so every
// load is in bounds; such keys are masked or never consumed.
__device__ inline void issue_tile(char *slot, const uint16_t *kt, int rmax, int rowstride, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int P = 128 * wave + 64 * i + lane;
    const int row = P >> 4;
    const uint16_t *src = kt + (int64_t)min(row, rmax) * rowstride + (((P & 15) ^ (row & 15)) * 8);
    __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)(slot + (128 * wave + 64 * i) * 16), 16, 0, 0);
  }
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

// RT: row tiles (of 32 rows) per wave.
// RT: full row tiles (of 32 rows) per wave.  SPLIT: there is one more row
// tile (4 RT + 1 in all), split into four 16 x 16 blocks per key tile, one
// per wave: wave v takes its rows 16 (v / 2) .. + 15 against the key tile's
// keys 16 (v % 2) .. + 15, with v_mfma_f32_16x16x32_bf16, so that no wave
// carries a whole extra tile (the slowest wave sets every step's pace).
template <int PASS, int RT, bool SPLIT = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(SPLIT ? (RT > 2 ? 1 : 2) : RT > 1 ? 1 : 4))) void score_kernel(ScoreParams p, SegTable t) {
  // The LDS ring: one array per slot, so that the compiler can tell a
  // slot being read from the slots that loads are landing in.
  __shared__ __attribute__((aligned(16))) char tile0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char tile1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char tile2[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char tile3[TILE_BYTES];
  extern __shared__ float red[];  // pass 2: [NW][key_block] partial sums

  const int blk = blockIdx.x;
  const int h = blockIdx.y;
  const int sb = blockIdx.z;
  const int64_t key0 = t.key_off[sb];
  const int L = (int)(t.key_off[sb + 1] - key0);
  // Keys key_begin + blk * key_block onwards, clipped to [key_begin,
  // key_end) of the launch (the whole prefix unless streaming).
  const int kend = min(L, p.key_end);
  const int kb0 = p.key_begin + blk * p.key_block;
  if (kb0 >= kend) return;  // the whole workgroup leaves together
  const int kb1 = min(kend, kb0 + p.key_block);
  const int seg = t.seg0 + sb * p.Hkv + h;
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
    lim[k] = row_limit((wave + NW * k) * 32 + lr, p, L);
    if constexpr (PASS == 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = (wave + NW * k) * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
        bias[k][i] = (k < my_rt) ? p.bias[(int64_t)seg * p.Rpad + row] : INFINITY;
      }
    }
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
    lim5 = row_limit(row, p, L);
    if constexpr (PASS == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) bias5[i] = p.bias[(int64_t)seg * p.Rpad + srow + 4 * s4 + i];
    }
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
  const int rowstride = p.Hkv * kHeadDim;  // elements between consecutive keys of one head
  const uint16_t *kblk = p.K + (key0 + kb0) * (int64_t)rowstride + (int64_t)h * kHeadDim;
  const int last = kb1 - 1 - kb0;  // block-relative index of the block's last key
  // LDS byte offset of this lane's operand chunk for k-step j: row lr, chunk 2j + hf, swizzled.
  const int rd_base = lr * ROWB;
  const int sw = lr & 15;

  // Tiles go straight from memory into a ring of PD = 4 LDS slots, three
  // tiles ahead of the one being consumed.  Every step issues exactly two
  // loads per wave (past the block they re-read its last key), so before
  // step t this wave has tiles t .. t + 2 in flight, and waiting until at
  // most 2 (PD - 2) loads remain means tile t has landed.
  auto tile_src = [&](int ti) { return kblk + (int64_t)(ti * KT) * rowstride; };
  issue_tile(tile0, tile_src(0), last, rowstride, wave, lane);
  issue_tile(tile1, tile_src(1), last - KT, rowstride, wave, lane);
  issue_tile(tile2, tile_src(2), last - 2 * KT, rowstride, wave, lane);

  // Consumes tile ti from `cur` after refilling `nxt` (the slot of tile
  // ti - 1) with tile ti + 3.
  auto step = [&](const int ti, const char *cur, char *nxt) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(kWaitTile);  // this wave's part of tile ti is in LDS
    __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0): this wave's reads of tile ti - 1 are done
    __builtin_amdgcn_s_barrier();           // every wave's part has landed; nxt is free
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    issue_tile(nxt, tile_src(ti + 3), last - (ti + 3) * KT, rowstride, wave, lane);
    if (ti >= ntile) return;  // padding step of the last group of four
    const char *slot = cur;
    const int i0 = kb0 + ti * KT;
    if (my_rt == 0) {  // this wave owns no rows (fewer than four row tiles in all)
      if constexpr (PASS == 2)
        if (hf == 0) red[wave * p.key_block + ti * KT + lr] = 0.0f;
      return;
    }

    f32x16 acc[RT];
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
    f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
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
    const bool need_mask = (i0 + KT - 1) > minlim;

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
          const int key = i0 + lr;
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
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = fast_exp2(fmaf(sacc[i], cl2, -bias5[i]));
          s5 += (need_mask && (i0 + skey + s16) > row_limit(srow + 4 * s4 + i, p, L)) ? 0.0f : v;
        }
        s5 += __shfl_xor(s5, 16);
        s5 += __shfl_xor(s5, 32);
        s += ((lr >> 4) == (wave & 1)) ? s5 : 0.0f;
      }
      if (hf == 0) red[wave * p.key_block + ti * KT + lr] = s;
    }
  };
  for (int t0 = 0; t0 < ntile; t0 += PD) {
    step(t0, tile0, tile3);
    step(t0 + 1, tile1, tile0);
    step(t0 + 2, tile2, tile1);
    step(t0 + 3, tile3, tile2);
  }
  // The last steps issued loads for tiles past the block that nobody
  // consumes; they write LDS, so drain them before the workgroup can end.
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  if constexpr (PASS == 2) {
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
    // block's per-row state; the blocks are merged by merge_kernel.
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

// Merge of the pass-1 block states of every (sequence, head) into the
// per-row bias = r + log2(Z) - log2(c_r) that pass 2 subtracts.  A separate
// launch: the kernel boundary makes every block's partials visible, with no
// per-workgroup cache write-backs.  Workgroup (row group of 16, segment):
// sixteen threads share a row, each merging every sixteenth block with 16
// loads in flight; the shares are combined in a fixed order through LDS.
constexpr int MERGE_ROWS = 16;
constexpr int MERGE_SPLIT = NT / MERGE_ROWS;

// FOLD (the streaming form, TideKV §4.2 with a bounded workspace): merge the
// block states of the step's keys [key_begin, key_end) and the running
// state `run` (unless this is the first step) back into `run` instead.
template <bool FOLD>
__global__ __launch_bounds__(NT) void merge_kernel(ScoreParams p, SegTable t, float2 *run, int first) {
  __shared__ float2 shares[MERGE_SPLIT][MERGE_ROWS];
  const int sl = blockIdx.y;  // local segment: sequence-major, head-minor
  const int sb = sl / p.Hkv;
  const int seg = t.seg0 + sl;
  const int L = (int)(t.key_off[sb + 1] - t.key_off[sb]);
  const int kend = min(L, p.key_end);
  const int nblk = FOLD ? ((kend > p.key_begin) ? (kend - p.key_begin + p.key_block - 1) / p.key_block : 0)
                        : (L + p.key_block - 1) / p.key_block;
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
  if constexpr (FOLD) {
    float2 *mine = run + (int64_t)seg * p.Rpad + row;
    if (!first) {
      const float2 prev = *mine;
      lse_merge(r, z, prev.x, prev.y);
    }
    *mine = make_float2(r, z);
    return;
  }
  const int wr = row / p.G;  // observation row: window rows 0 .. w-1, then the decode row
  float lc;                  // log2 of the row's weight c_r
  if (p.weighting == 1) {
    // c_r = 2^(lambda log2(e) (r - r_max)) / norm, relative position r = wr - (w - 1)
    lc = p.lam2 * (float)(wr - (p.w - 1) - p.has_decode) - p.log2norm;
  } else {
    float c = 1.0f;
    if (p.has_decode) c = (wr < p.w) ? (1.0f - p.alpha) : p.alpha;
    lc = (c > 0.0f) ? log2f(c) : -INFINITY;
  }
  float out = INFINITY;  // a row of weight 0 (or without visible keys) contributes nothing
  if (row < p.R && lc > -INFINITY && z > 0.0f) out = r + log2f(z) - lc;
  p.bias[(int64_t)seg * p.Rpad + row] = out;
}

template <int PASS>
hipError_t launch_pass(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s, size_t lds) {
  const dim3 grid(nblk, p.Hkv, t.nseq);
  const dim3 block(NT);
  if (p.nrt % NW == 1 && p.nrt > NW) {  // whole row tiles per wave plus a split one
    switch (p.nrt / NW) {
      case 1: hipLaunchKernelGGL((score_kernel<PASS, 1, true>), grid, block, lds, s, p, t); break;
      case 2: hipLaunchKernelGGL((score_kernel<PASS, 2, true>), grid, block, lds, s, p, t); break;
      default: hipLaunchKernelGGL((score_kernel<PASS, 3, true>), grid, block, lds, s, p, t); break;
    }
    return hipGetLastError();
  }
  const int rt = (p.nrt + NW - 1) / NW;
  switch (rt) {
    case 1: hipLaunchKernelGGL((score_kernel<PASS, 1>), grid, block, lds, s, p, t); break;
    case 2: hipLaunchKernelGGL((score_kernel<PASS, 2>), grid, block, lds, s, p, t); break;
    case 3: hipLaunchKernelGGL((score_kernel<PASS, 3>), grid, block, lds, s, p, t); break;
    default: hipLaunchKernelGGL((score_kernel<PASS, 4>), grid, block, lds, s, p, t); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_pass1(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  return launch_pass<1>(p, t, nblk, s, 0);
}

hipError_t launch_score_merge(const ScoreParams &p, const SegTable &t, hipStream_t s) {
  const dim3 grid((p.Rpad + MERGE_ROWS - 1) / MERGE_ROWS, t.nseq * p.Hkv);
  hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(NT), 0, s, p, t, (float2 *)nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_stream_stats(const ScoreParams &p, const SegTable &t, float2 *run, int first, hipStream_t s) {
  const dim3 grid((p.Rpad + MERGE_ROWS - 1) / MERGE_ROWS, t.nseq * p.Hkv);
  hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(NT), 0, s, p, t, run, first);
  return hipGetLastError();
}

hipError_t launch_score_pass2(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s) {
  return launch_pass<2>(p, t, nblk, s, (size_t)NW * p.key_block * sizeof(float));
}

}  // namespace kvsel
