// Internal declarations shared by the host side of libkvsel and its kernels.
// Not part of the public ABI (include/kvsel.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

constexpr int kHeadDim = 128;        // d supported by this build
constexpr int kMaxSeg = 64;          // (sequence, KV head) segments handled per launch
constexpr int kTile = 16;            // keys per MFMA tile and rows per row tile
constexpr int kRowTilesPerWave = 4;  // most row tiles (of 16 rows) held by one wave
constexpr int kMaxRows = 512;        // observation rows per KV head (G * w')
constexpr int kSelectThreads = 1024; // threads of the per-segment select workgroup
constexpr int kTicketBytes = kMaxSeg * 8;  // ticket header at the start of every workspace
constexpr int kMaxPoolKernel = 255;  // widest pool supported

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
  unsigned long long *tickets;  // arrival tickets of the launch's segments (fixed header of the workspace)
  int Hq, Hkv, G, w, wp, R, Rpad, nrt;
  int has_decode, causal;
  float cl2;                    // scale * log2(e)
  float alpha;
  int key_block;                // keys per workgroup in this pass
  int nblk1_max;                // pass 1 blocks per segment of the longest sequence
  int nrg, ks;                  // row groups and key splits (waves = nrg * ks)
  int rt;                       // row tiles per row group (1..4)
};

struct SelectParams {
  const float *scores;
  float *pooled;
  int32_t *idx;
  int Hkv;
  int pool;         // 0 none, 1 avg, 2 max
  int pool_kernel;  // odd
};

struct GatherParams {
  const int32_t *idx;
  const uint4 *K;   // rows of d bf16 = 16 x uint4
  const uint4 *V;
  uint4 *K_out;
  uint4 *V_out;
  int Hkv;
};

hipError_t launch_score_pass1(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
hipError_t launch_score_pass2(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t s);
hipError_t launch_pool_topk(const SelectParams &p, const SegTable &t, hipStream_t s);
hipError_t launch_gather(const GatherParams &p, const SegTable &t, hipStream_t s);

}  // namespace kvsel
