// Internal declarations shared by the host side of libkvsel and its kernels.
// Not part of the public ABI (include/kvsel.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvsel.h"

namespace kvsel {

constexpr int kHeadDim = 128;        // d supported by this build
constexpr int kMaxSeg = 64;          // (sequence, KV head) segments handled per launch
constexpr int kKeyTile = 32;         // keys per score tile (one 32x32 MFMA column block)
constexpr int kRowTile = 32;         // observation rows per row tile
constexpr int kScoreThreads = 256;   // threads (4 waves) of a score workgroup
constexpr int kMaxRows = 512;        // observation rows per KV head (G * w'): 16 row tiles, 4 per wave
constexpr int kMaxPoolKernel = 255;  // widest pool supported
constexpr int kSelectChunk = 2048;   // positions per pool / select workgroup
constexpr int kSelectBins = 8192;    // bins of the first radix digit (top 13 bits of an order key)
constexpr int kMaxChunks = 512;      // chunks per sequence, so L_b <= 2^20
// Selection tables built by pass 2 of kvsel_compress (pool and first-digit
// counting sort fused into the scoring): per block of kTabBlock positions,
// the exclusive prefix of the block's digit histogram and its order keys
// grouped by digit, plus each segment's whole histogram.
constexpr int kTabBlock = 256;       // positions per table block
constexpr int kTabBins = 2048;       // bins of the first digit
constexpr int kTabDigitShift = 16;   // a bin spans 2^16 order-key steps (1/128 of a factor 2 in value)
constexpr int kPoolHalo = 16;        // keys scored past each end of a pass-2 block for the pool (radius <= 16)
constexpr int kTabHistCopies = 8;    // copies of each segment's histogram (workgroup w adds to copy w mod 8, the
                                     // compute die it runs on, so that no count is contended across dies)

// Per-launch description of the sequences and segments a kernel works on.
// Travels by value in the kernel arguments, so no device-side tables are
// needed and launches can be captured into graphs.
struct SegTable {
  int32_t nseq;                 // sequences in this launch
  int32_t seq0;                 // global index of the first one
  int32_t seg0;                 // global index of its first (sequence, head) segment
  int32_t kmax;                 // largest kept count over the launch's segments
  int64_t key_off[kMaxSeg + 1]; // global key-row offset of each sequence, plus the end
  int64_t out_off[kMaxSeg];     // first output row of each local segment (sb * Hkv + h)
  int32_t keff[kMaxSeg];        // kept rows of each local segment
};

struct ScoreParams {
  const uint16_t *Q;            // bf16 [B][w'][Hq][d]
  const uint16_t *K;            // bf16 [sum L][Hkv][d]
  float *scores;                // pass 2 output (layout of the public ABI)
  float2 *partials;             // pass 1 per-block (ref, Z), [nseg][nblk1_max][Rpad]
  int Hq, Hkv, G, w, wp, R;
  int nrt;                      // row tiles of 32 rows
  int Rpad;                     // nrt * 32
  int has_decode, causal;
  float cl2;                    // scale * log2(e)
  float alpha;
  int weighting;                // 0: alpha weights; 1: exponential temporal weights
  float lam2;                   // weighting 1: lambda * log2(e)
  float log2norm;               // weighting 1: log2 of sum_r exp(lambda (r - r_max))
  int key_block;                // keys per workgroup in this pass (multiple of 32)
  int nblk1_max;                // pass 1 blocks per segment of the longest sequence
  int stat_block;               // pass 2: keys per pass-1 block state it merges (ceil(L / stat_block) per segment)
  int key_begin, key_end;       // keys of each sequence this launch covers (0, INT_MAX: all)
  int64_t out_stride;           // pass 2 output: 0 = the public layout; else floats per segment
  int out_origin;               //   and the key stored first in each segment's window
  // Pass 2 with selection tables (kvsel_compress): the pool of S over the
  // block (and kPoolHalo keys past each end), the pooled output and the
  // tables of each kTabBlock positions; `scores` may then be null.
  float *pooled;                // public layout
  uint16_t *tab;                // [nseg][ntab_max][kTabBins]: exclusive prefix of each block's digit histogram
  uint32_t *bucket;             // [nseg][ntab_max][kTabBlock]: each block's order keys grouped by digit
  uint32_t *seg_hist;           // [nseg][kTabHistCopies][kTabBins]: each segment's digit histogram, in
                                //   copies that add up to it (cleared by pass 1)
  int ntab_max;                 // table blocks of the longest sequence
  int pool, pool_r;             // pool kind (0 none, 1 avg, 2 max); half width (<= kPoolHalo)
  float pool_width;
  int sink, recent;
  float wsum;                   // sum of S over a segment's positions: G * sum_r c_r
  // Pass 2 with the pool in the streaming form of kvsel_compress (tab null):
  // the order keys of the pooled scores (select_key) of positions
  // step_origin onwards go to step_keys + seg * step_stride.
  uint32_t *step_keys;
  int64_t step_stride;
  int step_origin;
  // Pass 2 with the pool: workgroups with linear index in [young_from,
  // 2 young_from) (the second of two per compute unit) raise their waves'
  // priority for the first half of their key tiles; 0: off.  Set by the
  // launch from the device's compute units.
  int young_from;
};

// The mean query of every (sequence, observation row, KV head): the G query
// heads of the group averaged, rounded to bf16.
struct QueryMeanParams {
  const uint4 *Q;  // bf16 [B][w'][Hq][d], 16 uint4 per row of d = 128
  uint4 *Qm;       // bf16 [B][w'][Hkv][d]
  int Hq, Hkv, G;
  int items;       // B * w' * Hkv
};

struct SelectParams {
  const float *scores;
  float *pooled;
  int32_t *idx;
  uint16_t *tab_fine;    // [nseg][nchunk_max][kSelectBins]: exclusive prefix of each chunk's first-digit histogram
  uint16_t *tab_coarse;  // [nseg][nchunk_max][kSelectBins / 32]: every 32nd entry of tab_fine
  uint32_t *bucket;      // [nseg][nchunk_max][kSelectChunk]: each chunk's order keys grouped by first digit
  int nchunk_max;        // chunks of kSelectChunk positions in the longest sequence
  // Tables of the fused pass 2 (launch_select_blocks): tab_fine and bucket
  // then hold ScoreParams::tab and ::bucket.
  const uint32_t *seg_hist;
  int nblk_max;
  int Hkv;
  int pool;              // 0 none, 1 avg, 2 max
  int pool_kernel;       // odd
  int sink, recent;      // reserved positions: [0, sink) and [L - recent, L) of every sequence
  // Optional K/V compaction fused into the selection (K_out == nullptr: off).
  const uint4 *K;        // rows of d bf16 = 16 x uint4
  const uint4 *V;
  uint4 *K_out;
  uint4 *V_out;
};

// Warm-up profile: per sequence, the sum over KV heads of the scores.
struct ProfileParams {
  const float *scores;  // layout of the public ABI: segment (b, h) at Hkv * key_off[b] + h * L_b
  float *profile;       // [sum L], sequence b at key_off[b]
  int Hkv;
  int accumulate;       // 1: add to the profile; 0: overwrite it
};

// Kept importance: per segment, the sum of pooled[idx] over its kept positions.
struct MassParams {
  const float *pooled;  // layout of the public ABI
  const int32_t *idx;   // kept positions, segments at out_off
  float *mass;          // [segments][n_sizes]
  int Hkv;
  int n_sizes;
  int j;                // the column written by this launch
};

// Streaming selection: per segment a candidate row of lv floats, the running
// top-k values in [0, kslot) (ascending positions, -inf where unused) and
// this step's pooled values in [kslot, kslot + stream).
struct StreamParams {
  const float *S;         // pass-2 window: [nseg][S_stride], element 0 is key S_origin
  int64_t S_stride;
  int S_origin;
  float *cand;            // [nseg][lv]: this step's row (filled by init and pool, read by map)
  float *cand_next;       // [nseg][lv]: the next step's row (running part written by map)
  const int32_t *sel;     // selected slots of cand, per segment at the step plan's out_off
  const int32_t *pos_in;  // [nseg][kslot] positions of the running slots
  int32_t *pos_out;
  int lv, kslot, stream;
  int c0;                 // first key of this step
  int Hkv;
  int pool, pool_kernel;
  int sink, recent;
};

// The running top-k of the streaming form, one workgroup per segment: a
// row of lv order keys per segment holds the running set in slots
// [0, kslot) (its first min(keff, keys before c0) valid, positions in
// pos_in) and the step's keys in [kslot, kslot + stream) (positions c0 ..);
// the best keff of the valid ones, in slot order, become the next running
// set (keys_out, pos_out) or, at the last step, the result (idx).
struct StreamSelectParams {
  const uint32_t *keys_in;  // [nseg][lv]
  const int32_t *pos_in;    // [nseg][kslot]
  uint32_t *keys_out;       // [nseg][lv]: slots [0, kslot) written
  int32_t *pos_out;         // [nseg][kslot]
  int32_t *idx;             // last step: the public layout (SegTable::out_off)
  int lv, kslot, stream, c0, Hkv;
  float wsum;               // sum of S over a segment's positions (the first digit's centre)
  int last;                 // 1: write idx instead of keys_out / pos_out
};

struct GatherParams {
  const int32_t *idx;
  const uint4 *K;   // rows of d bf16 = 16 x uint4
  const uint4 *V;
  uint4 *K_out;
  uint4 *V_out;
  int Hkv;
};

// Sets kvsel_last_error's message (this thread) and returns s.
kvsel_status set_error(kvsel_status s, const char *msg);

hipError_t launch_query_mean(const QueryMeanParams &p, hipStream_t s);
hipError_t launch_profile(const ProfileParams &p, const SegTable &t, int64_t lmax, hipStream_t s);
hipError_t launch_tier_fill(int8_t *tier, int64_t n, hipStream_t s);
hipError_t launch_mass(const MassParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_tier_mark(const int32_t *idx, int8_t *tier, int label, const SegTable &t, hipStream_t s);
hipError_t launch_score_pass1(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
hipError_t launch_score_pass2(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
// Pass 2 with the pool and the selection tables (p.pooled, p.tab, ...);
// key_block a multiple of kTabBlock, pool radius <= kPoolHalo.
hipError_t launch_score_pass2_tables(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
// Pass 2 with the pool, writing the pooled scores' order keys
// (p.step_keys); key_block a multiple of kKeyTile, pool radius <= kPoolHalo.
hipError_t launch_score_pass2_keys(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
hipError_t launch_stream_select(const StreamSelectParams &p, const SegTable &t, hipStream_t s);
// Largest row (kslot + stream) launch_stream_select takes.
constexpr int kStreamRowMax = 16384;
hipError_t launch_stream_stats(const ScoreParams &p, const SegTable &t, float2 *run, int first, hipStream_t s);
hipError_t launch_stream_init(const StreamParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_stream_pool(const StreamParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_stream_map(const StreamParams &p, const SegTable &vt, hipStream_t s);
hipError_t launch_stream_final(const StreamParams &p, const SegTable &t, int32_t *idx, hipStream_t s);
hipError_t launch_pool_topk(const SelectParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_select_blocks(const SelectParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_gather(const GatherParams &p, const SegTable &t, hipStream_t s);

}  // namespace kvsel
