// Internal declarations shared by the host side of libkvsel and its kernels.
// Not part of the public ABI (include/kvsel.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// Resident scoring (both passes of a key block in one workgroup, the block's
// keys held in LDS between them).
constexpr int kResThreads = 256;     // four waves
constexpr int kResBlock = 256;       // keys per workgroup (= threads: one position each in the epilogue)
constexpr int kResHalo = 16;         // keys scored on each side of a block for the pool (pool radius <= 16)
constexpr int kResMaxRows = 128;     // observation rows per KV head (a row tile of 32 per wave)
constexpr int kResBins = 2048;       // bins of the selection's first digit
constexpr int kResDigitShift = 16;   // a bin spans 2^16 order-key steps (1/128 of a factor 2 in value)
constexpr int kResSpinCap = 8192;    // polls of a block's wait for its segment before it computes what is missing

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
  float *bias;                  // pass 1 result per row, [nseg][Rpad]
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
  int key_begin, key_end;       // keys of each sequence this launch covers (0, INT_MAX: all)
  int64_t out_stride;           // pass 2 output: 0 = the public layout; else floats per segment
  int out_origin;               //   and the key stored first in each segment's window
};

// The mean query of every (sequence, observation row, KV head): the G query
// heads of the group averaged, rounded to bf16.
struct QueryMeanParams {
  const uint4 *Q;  // bf16 [B][w'][Hq][d], 16 uint4 per row of d = 128
  uint4 *Qm;       // bf16 [B][w'][Hkv][d]
  int Hq, Hkv, G;
  int items;       // B * w' * Hkv
};

// Words of the resident scoring's synchronisation area (64-bit):
//   [0]                           T, the call token; the kernel that runs
//                                 after the scoring sets it to T + 1 for
//                                 the next call
//   [1]                           the T the last scoring ran with
//   [2 + seg]                     == T + 1: segment seg's histogram lacks the
//                                 counts of blocks that stopped waiting
//   [2 + nseg + seg]              == T + 1: segment seg's row biases are
//                                 published
//   [2 + 2 nseg + seg]            == T + 1: ... by a merger that saw every
//                                 block publish
//   [2 + 3 nseg + sl * nblk + b]  == T + 1: block b of local segment sl has
//                                 published its row statistics
// Flags from earlier calls hold other tokens, so nothing needs clearing.
constexpr int kSyncFlags = 2;
constexpr int kSyncIncomplete = kSyncFlags;

// The fused scoring of kvsel_compress: per block of kResBlock keys of one
// (sequence, KV head) segment, pass 1, the segment's statistics merge,
// pass 2 over the same keys (still in LDS), the pool and the block's
// first-digit counting sort.
struct ResidentParams {
  const uint16_t *Q;     // bf16 [B][w'][Hq][d] (mean queries [B][w'][Hkv][d] with G = 1)
  const uint16_t *K;     // bf16 [sum L][Hkv][d]
  float *scores;         // optional: S in the public layout (nullptr: not written)
  float *pooled;         // pooled scores, public layout
  uint16_t *tab;         // [nseg][nblk_max][kResBins]: exclusive prefix of each block's digit histogram
  uint32_t *bucket;      // [nseg][nblk_max][kResBlock]: each block's order keys grouped by digit
  uint32_t *seg_hist;    // [nseg][kResBins]: each segment's digit histogram (its blocks clear it)
  float *lse;            // [nseg][nblk_max][Rp]: per block and row, log2 of the sum of 2^(s log2 e)
  float *biasg;          // [nseg][Rp]: the row biases, published by each segment's first block
  float *refg;           // [nseg][nblk][Rp]: each block's reference logit per row (its e = 2^(x - ref))
  uint64_t *sync;        // call tokens and flags (res_sync below)
  int nseg;              // segments of the whole problem (global indices)
  int Hq, Hkv, G, w, wp, R, Rp;  // Rp: rows rounded up to 16
  int has_decode, causal;
  float cl2, alpha;
  int weighting;
  float lam2, log2norm;
  float wsum;            // sum of S over a segment's positions: G * sum_r c_r
  int pool, pool_r;      // pool kind; half width (<= kResHalo)
  float pool_width;
  int sink, recent;
  int nblk_max;          // blocks of the longest sequence
  int spin_cap;          // polls before a block stops waiting (0: never wait)
  int tables;            // 1: pool, pooled output and selection tables; 0: scores only
};

struct SelectParams {
  const float *scores;
  float *pooled;
  int32_t *idx;
  uint16_t *tab_fine;    // [nseg][nchunk_max][kSelectBins]: exclusive prefix of each chunk's first-digit histogram
  uint16_t *tab_coarse;  // [nseg][nchunk_max][kSelectBins / 32]: every 32nd entry of tab_fine
  uint32_t *bucket;      // [nseg][nchunk_max][kSelectChunk]: each chunk's order keys grouped by first digit
  int nchunk_max;        // chunks of kSelectChunk positions in the longest sequence
  // Tables of the resident scoring (launch_select_blocks): tab_fine and
  // bucket then hold ResidentParams::tab and ::bucket.
  const uint32_t *seg_hist;
  uint64_t *sync;        // ResidentParams::sync
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

struct GatherParams {
  const int32_t *idx;
  const uint4 *K;   // rows of d bf16 = 16 x uint4
  const uint4 *V;
  uint4 *K_out;
  uint4 *V_out;
  int Hkv;
};

hipError_t launch_query_mean(const QueryMeanParams &p, hipStream_t s);
hipError_t launch_profile(const ProfileParams &p, const SegTable &t, int64_t lmax, hipStream_t s);
hipError_t launch_tier_fill(int8_t *tier, int64_t n, hipStream_t s);
hipError_t launch_mass(const MassParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_tier_mark(const int32_t *idx, int8_t *tier, int label, const SegTable &t, hipStream_t s);
hipError_t launch_score_pass1(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
hipError_t launch_score_merge(const ScoreParams &p, const SegTable &t, hipStream_t s);  // key_block = pass 1's
hipError_t launch_score_pass2(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
hipError_t launch_stream_stats(const ScoreParams &p, const SegTable &t, float2 *run, int first, hipStream_t s);
hipError_t launch_stream_init(const StreamParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_stream_pool(const StreamParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_stream_map(const StreamParams &p, const SegTable &vt, hipStream_t s);
hipError_t launch_stream_final(const StreamParams &p, const SegTable &t, int32_t *idx, hipStream_t s);
hipError_t launch_pool_topk(const SelectParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_resident_bump(uint64_t *sync, hipStream_t s);
hipError_t launch_resident(const ResidentParams &p, const SegTable &t, int items, hipStream_t s);
hipError_t launch_select_blocks(const SelectParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_gather(const GatherParams &p, const SegTable &t, hipStream_t s);

}  // namespace kvsel
