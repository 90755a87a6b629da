// Host-only stand-ins for the GPU side of libkvsel, for the sanitized CPU
// build of the host library (kvsel_api.cpp): a device that reports gfx950,
// and kernel launches that run nothing but check, from each launch's
// parameters and the kernels' indexing, that every array the kernel would
// touch lies inside one of the buffers the driver registered (the caller's
// inputs, outputs and workspace).  A layout or offset mistake in the host
// code that would send a kernel past a buffer shows up here as a failure.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "kvsel_internal.h"
#include "registry.h"

namespace {

struct Buf {
  const char *base;
  size_t bytes;
  const char *name;
};
std::vector<Buf> g_bufs;
int g_failures = 0;
int g_launches = 0;

void need(const void *p, int64_t bytes, const char *what) {
  if (bytes <= 0) return;
  if (!p) {
    std::fprintf(stderr, "FAIL %s: null pointer for %lld bytes\n", what, (long long)bytes);
    ++g_failures;
    return;
  }
  const char *c = static_cast<const char *>(p);
  for (const Buf &b : g_bufs)
    if (c >= b.base && c + bytes <= b.base + b.bytes) return;
  std::fprintf(stderr, "FAIL %s: [%p, +%lld) is inside no registered buffer\n", what, p, (long long)bytes);
  ++g_failures;
}

void expect(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s\n", what);
    ++g_failures;
  }
}

using namespace kvsel;

int64_t seg_end(const SegTable &t, int Hkv) { return t.seg0 + (int64_t)t.nseq * Hkv; }
int64_t key_end(const SegTable &t) { return t.key_off[t.nseq]; }
int64_t lmax(const SegTable &t) {
  int64_t m = 0;
  for (int i = 0; i < t.nseq; ++i) m = std::max<int64_t>(m, t.key_off[i + 1] - t.key_off[i]);
  return m;
}
int64_t out_rows(const SegTable &t, int Hkv) {
  int64_t m = 0;
  for (int64_t s = 0; s < (int64_t)t.nseq * Hkv; ++s) m = std::max<int64_t>(m, t.out_off[s] + t.keff[s]);
  return m;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

void score_common(const ScoreParams &p, const SegTable &t, int nblk, int pass) {
  need(p.Q, (int64_t)(t.seq0 + t.nseq) * p.wp * p.Hq * kHeadDim * 2, "score: Q");
  need(p.K, key_end(t) * p.Hkv * kHeadDim * 2, "score: K");
  need(p.partials, seg_end(t, p.Hkv) * p.nblk1_max * p.Rpad * 8, "score: block states");
  expect(p.key_block % kKeyTile == 0 && p.key_block > 0, "score: key_block a positive multiple of 32");
  const int64_t last = std::min<int64_t>(lmax(t), p.key_end);
  expect((int64_t)p.key_begin + (int64_t)nblk * p.key_block >= last, "score: the grid covers every key");
  if (pass == 1) {
    expect(p.key_begin % kKeyTile == 0, "pass 1: blocks start on a key tile");
    expect(nblk <= p.nblk1_max, "pass 1: block index within the block states");
  } else {
    expect(ceil_div(lmax(t), p.stat_block) <= p.nblk1_max, "pass 2: merged block states within the workspace");
  }
}

}  // namespace

void reg_clear() { g_bufs.clear(); }
void reg_add(const void *p, size_t bytes, const char *name) {
  g_bufs.push_back({static_cast<const char *>(p), bytes, name});
}
int reg_failures() { return g_failures; }
int reg_launches() { return g_launches; }

// ---- the device
hipError_t hipGetDevice(int *dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *prop, int) {
  std::memset(prop, 0, sizeof(*prop));
  std::strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  return hipSuccess;
}
const char *hipGetErrorString(hipError_t) { return "stub"; }

// ---- the launches
namespace kvsel {

hipError_t launch_query_mean(const QueryMeanParams &p, hipStream_t) {
  ++g_launches;
  const int64_t rows = p.items / p.Hkv;  // B * w'
  need(p.Q, rows * p.Hq * kHeadDim * 2, "query mean: Q");
  need(p.Qm, (int64_t)p.items * kHeadDim * 2, "query mean: mean queries");
  return hipSuccess;
}

hipError_t launch_score_pass1(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t) {
  ++g_launches;
  score_common(p, t, nblk, 1);
  if (p.seg_hist) need(p.seg_hist, seg_end(t, p.Hkv) * kTabHistCopies * kTabBins * 4, "pass 1: histograms");
  return hipSuccess;
}

hipError_t launch_score_pass2(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t) {
  ++g_launches;
  score_common(p, t, nblk, 2);
  if (p.out_stride > 0) {
    expect(p.key_begin >= p.out_origin, "pass 2: window starts at or after its origin");
    const int64_t last = std::min<int64_t>(lmax(t), p.key_end);
    expect(last - p.out_origin <= p.out_stride, "pass 2: window holds the keys it is given");
    need(p.scores, seg_end(t, p.Hkv) * p.out_stride * 4, "pass 2: score windows");
  } else {
    need(p.scores, key_end(t) * p.Hkv * 4, "pass 2: scores");
  }
  return hipSuccess;
}

hipError_t launch_score_pass2_tables(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t) {
  ++g_launches;
  score_common(p, t, nblk, 2);
  expect(p.key_block % kTabBlock == 0, "pass 2 tables: whole table blocks");
  expect(p.pool_r >= 0 && p.pool_r <= kPoolHalo, "pass 2 tables: pool within the halo");
  expect(ceil_div(lmax(t), kTabBlock) <= p.ntab_max, "pass 2 tables: table blocks within the workspace");
  if (p.scores) need(p.scores, key_end(t) * p.Hkv * 4, "pass 2 tables: scores");
  need(p.pooled, key_end(t) * p.Hkv * 4, "pass 2 tables: pooled");
  need(p.tab, seg_end(t, p.Hkv) * p.ntab_max * kTabBins * 2, "pass 2 tables: prefix tables");
  need(p.bucket, seg_end(t, p.Hkv) * p.ntab_max * kTabBlock * 4, "pass 2 tables: buckets");
  need(p.seg_hist, seg_end(t, p.Hkv) * kTabHistCopies * kTabBins * 4, "pass 2 tables: histograms");
  return hipSuccess;
}

hipError_t launch_score_pass2_keys(const ScoreParams &p, const SegTable &t, int nblk, hipStream_t) {
  ++g_launches;
  score_common(p, t, nblk, 2);
  expect(p.pool_r >= 0 && p.pool_r <= kPoolHalo, "pass 2 keys: pool within the halo");
  expect(p.key_begin >= p.step_origin, "pass 2 keys: window starts at or after its origin");
  const int64_t last = std::min<int64_t>(lmax(t), p.key_end);
  expect(last - p.step_origin <= p.step_stride, "pass 2 keys: a row holds the step");
  need(p.step_keys, ((seg_end(t, p.Hkv) - 1) * p.step_stride + (last - p.step_origin)) * 4, "pass 2 keys: rows");
  return hipSuccess;
}

hipError_t launch_stream_select(const StreamSelectParams &p, const SegTable &t, hipStream_t) {
  ++g_launches;
  expect(p.lv % 4 == 0 && p.kslot % 4 == 0 && p.kslot + p.stream <= p.lv && p.lv <= kStreamRowMax,
         "streaming selection: row layout");
  expect(t.kmax <= p.kslot, "streaming selection: running slots hold every budget");
  need(p.keys_in, seg_end(t, p.Hkv) * p.lv * 4, "streaming selection: rows in");
  if (p.kslot > 0) need(p.pos_in, seg_end(t, p.Hkv) * p.kslot * 4, "streaming selection: positions in");
  if (p.last) {
    need(p.idx, out_rows(t, p.Hkv) * 4, "streaming selection: kept positions");
  } else {
    need(p.keys_out, seg_end(t, p.Hkv) * p.lv * 4, "streaming selection: rows out");
    if (p.kslot > 0) need(p.pos_out, seg_end(t, p.Hkv) * p.kslot * 4, "streaming selection: positions out");
  }
  return hipSuccess;
}

hipError_t launch_stream_stats(const ScoreParams &p, const SegTable &t, float2 *run, int, hipStream_t) {
  ++g_launches;
  need(p.partials, seg_end(t, p.Hkv) * p.nblk1_max * p.Rpad * 8, "fold: block states");
  need(run, seg_end(t, p.Hkv) * p.Rpad * 8, "fold: running states");
  return hipSuccess;
}

static void rows_out(const SegTable &t, int Hkv, const void *idx, const void *K, const void *V, const void *Ko,
                     const void *Vo, const char *what) {
  const int64_t rows = out_rows(t, Hkv);
  if (rows == 0) return;
  need(idx, rows * 4, what);
  if (Ko) {
    need(K, key_end(t) * Hkv * kHeadDim * 2, what);
    need(V, key_end(t) * Hkv * kHeadDim * 2, what);
    need(Ko, rows * kHeadDim * 2, what);
    need(Vo, rows * kHeadDim * 2, what);
  }
}

hipError_t launch_pool_topk(const SelectParams &p, const SegTable &t, hipStream_t) {
  ++g_launches;
  expect(ceil_div(lmax(t), kSelectChunk) <= p.nchunk_max, "pool/top-k: chunks within the workspace");
  need(p.scores, key_end(t) * p.Hkv * 4, "pool/top-k: scores");
  need(p.pooled, key_end(t) * p.Hkv * 4, "pool/top-k: pooled");
  need(p.tab_fine, seg_end(t, p.Hkv) * p.nchunk_max * kSelectBins * 2, "pool/top-k: prefix tables");
  need(p.tab_coarse, seg_end(t, p.Hkv) * p.nchunk_max * (kSelectBins / 32) * 2, "pool/top-k: coarse tables");
  need(p.bucket, seg_end(t, p.Hkv) * p.nchunk_max * kSelectChunk * 4, "pool/top-k: buckets");
  rows_out(t, p.Hkv, p.idx, p.K, p.V, p.K_out, p.V_out, "pool/top-k: kept rows");
  return hipSuccess;
}

hipError_t launch_select_blocks(const SelectParams &p, const SegTable &t, hipStream_t) {
  ++g_launches;
  expect(ceil_div(lmax(t), kTabBlock) <= p.nblk_max, "block selection: table blocks within the workspace");
  expect(ceil_div(lmax(t), kSelectChunk) <= kMaxChunks, "block selection: chunks within the launch limit");
  need(p.pooled, key_end(t) * p.Hkv * 4, "block selection: pooled");
  need(p.tab_fine, seg_end(t, p.Hkv) * p.nblk_max * kTabBins * 2, "block selection: prefix tables");
  need(p.bucket, seg_end(t, p.Hkv) * p.nblk_max * kTabBlock * 4, "block selection: buckets");
  need(p.seg_hist, seg_end(t, p.Hkv) * kTabHistCopies * kTabBins * 4, "block selection: histograms");
  rows_out(t, p.Hkv, p.idx, p.K, p.V, p.K_out, p.V_out, "block selection: kept rows");
  return hipSuccess;
}

hipError_t launch_gather(const GatherParams &p, const SegTable &t, hipStream_t) {
  ++g_launches;
  rows_out(t, p.Hkv, p.idx, p.K, p.V, p.K_out, p.V_out, "gather: rows");
  return hipSuccess;
}

hipError_t launch_profile(const ProfileParams &p, const SegTable &t, int64_t, hipStream_t) {
  ++g_launches;
  need(p.scores, key_end(t) * p.Hkv * 4, "profile: scores");
  need(p.profile, key_end(t) * 4, "profile: profile");
  return hipSuccess;
}

hipError_t launch_tier_fill(int8_t *tier, int64_t n, hipStream_t) {
  ++g_launches;
  need(tier, n, "tiers: fill");
  return hipSuccess;
}

hipError_t launch_tier_mark(const int32_t *idx, int8_t *tier, int, const SegTable &t, hipStream_t) {
  ++g_launches;
  need(idx, out_rows(t, 1) * 4, "tiers: ranked positions");
  need(tier, key_end(t), "tiers: labels");
  return hipSuccess;
}

hipError_t launch_mass(const MassParams &p, const SegTable &t, hipStream_t) {
  ++g_launches;
  need(p.pooled, key_end(t) * p.Hkv * 4, "mass: pooled");
  need(p.idx, out_rows(t, p.Hkv) * 4, "mass: kept positions");
  need(p.mass, seg_end(t, p.Hkv) * p.n_sizes * 4, "mass: output");
  expect(p.j >= 0 && p.j < p.n_sizes, "mass: column within the output");
  return hipSuccess;
}

static void stream_common(const StreamParams &p, const SegTable &t, const char *what) {
  need(p.cand, seg_end(t, p.Hkv) * p.lv * 4, what);
  expect(p.kslot + p.stream <= p.lv, "streaming: a candidate row holds the running slots and one step");
}

hipError_t launch_stream_init(const StreamParams &p, const SegTable &t, hipStream_t) {
  ++g_launches;
  stream_common(p, t, "streaming init: candidates");
  return hipSuccess;
}

hipError_t launch_stream_pool(const StreamParams &p, const SegTable &t, hipStream_t) {
  ++g_launches;
  stream_common(p, t, "streaming pool: candidates");
  need(p.S, seg_end(t, p.Hkv) * p.S_stride * 4, "streaming pool: score windows");
  return hipSuccess;
}

hipError_t launch_stream_map(const StreamParams &p, const SegTable &vt, hipStream_t) {
  ++g_launches;
  stream_common(p, vt, "streaming map: candidates");
  need(p.cand_next, seg_end(vt, p.Hkv) * p.lv * 4, "streaming map: next candidates");
  need(p.pos_in, seg_end(vt, p.Hkv) * p.kslot * 4, "streaming map: positions in");
  need(p.pos_out, seg_end(vt, p.Hkv) * p.kslot * 4, "streaming map: positions out");
  return hipSuccess;
}

hipError_t launch_stream_final(const StreamParams &p, const SegTable &t, int32_t *idx, hipStream_t) {
  ++g_launches;
  need(p.pos_in, seg_end(t, p.Hkv) * p.kslot * 4, "streaming final: positions");
  need(idx, out_rows(t, p.Hkv) * 4, "streaming final: kept positions");
  return hipSuccess;
}

}  // namespace kvsel
