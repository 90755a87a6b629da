// Host side of libkvsel: validation, planning, workspace layout and kernel
// launches behind the C ABI declared in include/kvsel.h.
#include "kvsel.h"
#include "kvsel_internal.h"

#include <atomic>
#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>


#define KVSEL_API extern "C" __attribute__((visibility("default")))

namespace {

using namespace kvsel;

thread_local std::string g_last_error;

kvsel_status fail(kvsel_status s, const std::string &msg) {
  g_last_error = msg;
  return s;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Everything the launches need, derived from a validated kvsel_problem.
struct Plan {
  int B, Hq, Hkv, G, w, wp, R, nrt, Rpad;
  int has_decode, causal, pool, pool_kernel;
  float alpha, cl2;
  int weighting = 0, sink = 0, recent = 0;
  int gqa = 0;          // KVSEL_GQA_MEAN_QUERY: Hq and G below describe the mean queries
  // Streaming (bounded workspace): keys per step, pool half width, running
  // top-k slots per segment, candidate row length, pass-1 blocks per step.
  int stream = 0, halo = 0, kslot = 0, lv = 0, nblk1_c = 0;
  size_t off_run = 0, off_sbuf = 0, off_cand[2] = {0, 0}, off_candp = 0, off_selidx = 0, off_pos[2] = {0, 0};
  int Hq_in = 0, G_in = 0;  // the caller's query heads and group size
  size_t off_qmean = 0;
  float lam2 = 0.0f, log2norm = 0.0f;
  std::vector<int64_t> seq_off;  // B + 1
  std::vector<int32_t> keff;     // B * Hkv
  std::vector<int64_t> out_off;  // B * Hkv + 1
  int64_t Lmax = 0;
  int kb1 = 0, kb2 = 0, nblk1_max = 0, nblk2_max = 0;
  int nchunk_max = 0;
  size_t off_partials = 0, off_scores = 0, off_pooled = 0, ws_bytes = 0;
  size_t off_tfine = 0, off_tcoarse = 0, off_bucket = 0;
  // kvsel_compress with the pool and the selection's first steps fused into
  // pass 2 (pools up to 33 wide): pass 2's key blocks in whole table blocks
  // of kTabBlock positions, the tables and the per-segment histograms.
  bool fused = false;
  int kb2t = 0, ntab_max = 0;
  size_t off_thist = 0, off_ttab = 0, off_tbucket = 0;
  // The fused streaming form (pools up to 2 kPoolHalo + 1 wide, running
  // rows up to kStreamRowMax): pass 2's key block per step, and two rows of
  // order keys and two of running positions per segment.
  bool sfused = false;
  int kb2s = 0;
  size_t off_skeys[2] = {0, 0}, off_spos[2] = {0, 0};
};

// Pass-1 block states per segment in the fused streaming form: a bound
// independent of the prefix length.
constexpr int kStreamStates = 64;

// Test hook read from the environment: KVSEL_UNFUSED=1 sends kvsel_compress
// through pass 2 without tables, then the separate pool and selection
// launches (the path of pools wider than 33), so that tests can compare the
// two.
bool env_unfused() {
  const char *e = std::getenv("KVSEL_UNFUSED");
  return e && e[0] == '1';
}

int auto_key_block(int64_t head_keys, int64_t cap) {
  // Aim for about 512 workgroups (two per compute unit) over the launch,
  // in whole 32-key tiles, at least two tiles per workgroup.  Larger blocks
  // load each head's queries fewer times, and a launch then leaves room for
  // another layer's kernels on other streams; 512 measured faster than 1024
  // and 256 both alone and with four layers in flight.
  const int64_t wgs = 512;
  int64_t kb = (head_keys + wgs - 1) / wgs;
  kb = (kb + kKeyTile - 1) / kKeyTile * kKeyTile;
  kb = std::max<int64_t>(kb, 2 * kKeyTile);
  kb = std::min<int64_t>(kb, cap);
  return (int)kb;
}

// Workspace of the streaming form (TideKV §4.2's bounded temporary memory):
// every part is sized by the keys per step, the budgets and the rows, never
// by the prefix length.
kvsel_status plan_streaming(const kvsel_problem *p, Plan &P) {
  const size_t nseg = (size_t)P.B * P.Hkv;
  P.stream = p->stream_keys;
  P.halo = (P.pool == KVSEL_POOL_NONE) ? 0 : (P.pool_kernel - 1) / 2;
  int32_t kmax = 0;
  for (int32_t k : P.keff) kmax = std::max(kmax, k);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const int kslot4 = (kmax + 3) / 4 * 4;
  P.sfused = P.halo <= kPoolHalo && (int64_t)kslot4 + P.stream <= kStreamRowMax && !env_unfused();
  if (P.sfused) {
    // Pass 1 runs once over the whole prefix with at most kStreamStates
    // block states per segment: blocks of the whole-prefix size, or longer
    // when the prefix needs more than kStreamStates of them.
    const int64_t span = (P.Lmax + kStreamStates - 1) / kStreamStates;
    P.kb1 = (int)std::max<int64_t>(P.kb1, (span + kKeyTile - 1) / kKeyTile * kKeyTile);
    P.nblk1_max = kStreamStates;  // the states' stride: the same workspace for every prefix length
    P.kb2s = auto_key_block((int64_t)P.stream * P.B * P.Hkv, 2048);
    P.kslot = kslot4;
    P.lv = kslot4 + P.stream;
    P.off_partials = take(nseg * P.nblk1_max * P.Rpad * sizeof(float2));
    P.off_run = take(nseg * P.Rpad * sizeof(float2));
    for (int i = 0; i < 2; ++i) P.off_skeys[i] = take(nseg * P.lv * sizeof(uint32_t));
    for (int i = 0; i < 2; ++i) P.off_spos[i] = take(nseg * std::max(4, P.kslot) * sizeof(int32_t));
    P.off_qmean = off;
    if (P.gqa == KVSEL_GQA_MEAN_QUERY) take((size_t)P.B * P.wp * P.Hkv * p->d * sizeof(uint16_t));
    P.off_scores = P.off_pooled = 0;  // no whole-prefix buffers in this form
    P.ws_bytes = off;
    return KVSEL_OK;
  }
  P.kslot = kmax;
  const int64_t lv = (int64_t)P.kslot + P.stream;
  if (lv > (int64_t)kMaxChunks * kSelectChunk)
    return fail(KVSEL_EUNSUPPORTED, "stream_keys plus the largest budget exceed 2^20");
  P.lv = (int)lv;
  // A step has fewer keys than a whole prefix; blocks of at least 128 keys
  // keep each workgroup's query loads small next to its key loads.
  const int64_t step_keys = (int64_t)P.stream * P.B * P.Hkv;
  P.kb1 = std::max(128, auto_key_block(step_keys, 4096));
  if (p->key_chunk > 0) P.kb1 = std::min(P.kb1, p->key_chunk);  // the caller's chunk bounds a block
  P.kb2 = std::max(128, auto_key_block(step_keys, 2048));
  P.nblk1_c = (P.stream + P.kb1 - 1) / P.kb1;
  P.nblk1_max = P.nblk1_c;
  P.nchunk_max = (P.lv + kSelectChunk - 1) / kSelectChunk;
  P.off_partials = take(nseg * P.nblk1_c * P.Rpad * sizeof(float2));
  P.off_run = take(nseg * P.Rpad * sizeof(float2));
  P.off_sbuf = take(nseg * ((size_t)P.stream + 2 * P.halo) * sizeof(float));
  P.off_cand[0] = take(nseg * P.lv * sizeof(float));
  P.off_cand[1] = take(nseg * P.lv * sizeof(float));
  P.off_candp = take(nseg * P.lv * sizeof(float));
  P.off_selidx = take(nseg * std::max(1, P.kslot) * sizeof(int32_t));
  P.off_pos[0] = take(nseg * std::max(1, P.kslot) * sizeof(int32_t));
  P.off_pos[1] = take(nseg * std::max(1, P.kslot) * sizeof(int32_t));
  const size_t nchunks = nseg * (size_t)P.nchunk_max;
  P.off_tfine = take(nchunks * kSelectBins * sizeof(uint16_t));
  P.off_tcoarse = take(nchunks * (kSelectBins / 32) * sizeof(uint16_t));
  P.off_bucket = take(nchunks * kSelectChunk * sizeof(uint32_t));
  P.off_qmean = off;
  if (P.gqa == KVSEL_GQA_MEAN_QUERY) take((size_t)P.B * P.wp * P.Hkv * p->d * sizeof(uint16_t));
  P.off_scores = P.off_pooled = 0;  // no whole-prefix buffers in this form
  P.ws_bytes = off;
  return KVSEL_OK;
}

kvsel_status make_plan(const kvsel_problem *p, Plan &P) {
  if (!p) return fail(KVSEL_EINVAL, "problem pointer is NULL");
  if (p->batch < 1) return fail(KVSEL_EINVAL, "batch must be >= 1");
  if (p->Hkv < 1 || p->Hq < 1) return fail(KVSEL_EINVAL, "Hq and Hkv must be >= 1");
  if (p->Hq % p->Hkv != 0) return fail(KVSEL_EINVAL, "Hq must be a multiple of Hkv");
  if (p->d < 1) return fail(KVSEL_EINVAL, "d must be >= 1");
  if (p->w < 1) return fail(KVSEL_EINVAL, "w must be >= 1");
  if (p->has_decode != 0 && p->has_decode != 1) return fail(KVSEL_EINVAL, "has_decode must be 0 or 1");
  if (p->causal != 0 && p->causal != 1) return fail(KVSEL_EINVAL, "causal must be 0 or 1");
  if (p->has_decode && !(p->alpha >= 0.0f && p->alpha <= 1.0f)) return fail(KVSEL_EINVAL, "alpha must lie in [0, 1]");
  if (!std::isfinite(p->scale)) return fail(KVSEL_EINVAL, "scale must be finite");
  if (p->pool < KVSEL_POOL_NONE || p->pool > KVSEL_POOL_MAX) return fail(KVSEL_EINVAL, "unknown pool kind");
  if (p->pool != KVSEL_POOL_NONE && (p->pool_kernel < 1 || p->pool_kernel % 2 == 0))
    return fail(KVSEL_EINVAL, "pool_kernel must be odd and >= 1");
  if (p->pool != KVSEL_POOL_NONE && p->pool_kernel > kMaxPoolKernel)
    return fail(KVSEL_EUNSUPPORTED, "pool_kernel wider than 255");
  if (p->key_chunk < 0 || p->key_chunk % kKeyTile != 0)
    return fail(KVSEL_EINVAL, "key_chunk must be 0 or a positive multiple of 32");
  if (!p->budgets_h && p->k < 0) return fail(KVSEL_EINVAL, "k must be >= 0");
  if (p->weighting != KVSEL_WEIGHT_ALPHA && p->weighting != KVSEL_WEIGHT_EXP)
    return fail(KVSEL_EINVAL, "unknown weighting");
  if (p->weighting == KVSEL_WEIGHT_EXP && !(std::isfinite(p->lambda) && p->lambda >= 0.0f))
    return fail(KVSEL_EINVAL, "lambda must be finite and >= 0");
  if (p->sink_tokens < 0 || p->recent_tokens < 0) return fail(KVSEL_EINVAL, "sink_tokens and recent_tokens must be >= 0");
  if (p->gqa != KVSEL_GQA_SUM && p->gqa != KVSEL_GQA_MEAN_QUERY) return fail(KVSEL_EINVAL, "unknown gqa");
  if (p->stream_keys < 0 || p->stream_keys % kSelectChunk != 0)
    return fail(KVSEL_EINVAL, "stream_keys must be 0 or a positive multiple of 2048");

  P.B = p->batch;
  P.Hq = p->Hq;
  P.Hkv = p->Hkv;
  P.G = p->Hq / p->Hkv;
  P.Hq_in = P.Hq;
  P.G_in = P.G;
  P.gqa = p->gqa;
  if (P.gqa == KVSEL_GQA_MEAN_QUERY) {  // the kernels score one mean query per KV head
    P.Hq = P.Hkv;
    P.G = 1;
  }
  P.w = p->w;
  P.wp = p->w + p->has_decode;
  P.seq_off.assign(P.B + 1, 0);
  if (p->seq_offsets_h) {
    if (p->seq_offsets_h[0] != 0) return fail(KVSEL_EINVAL, "seq_offsets_h[0] must be 0");
    for (int b = 0; b < P.B; ++b) {
      const int64_t Lb = p->seq_offsets_h[b + 1] - p->seq_offsets_h[b];
      if (Lb < 1) return fail(KVSEL_EINVAL, "every sequence needs at least one key (seq_offsets_h must increase)");
      P.seq_off[b + 1] = p->seq_offsets_h[b + 1];
    }
  } else {
    if (p->L < 1) return fail(KVSEL_EINVAL, "L must be >= 1");
    for (int b = 0; b < P.B; ++b) P.seq_off[b + 1] = P.seq_off[b] + p->L;
  }
  for (int b = 0; b < P.B; ++b) {
    const int64_t Lb = P.seq_off[b + 1] - P.seq_off[b];
    if (Lb > (int64_t)kMaxChunks * kSelectChunk) return fail(KVSEL_EUNSUPPORTED, "sequence longer than 2^20 keys");
    if (p->w > Lb) return fail(KVSEL_EINVAL, "w must not exceed any sequence length");
    P.Lmax = std::max(P.Lmax, Lb);
  }
  P.keff.assign((size_t)P.B * P.Hkv, 0);
  P.out_off.assign((size_t)P.B * P.Hkv + 1, 0);
  for (int b = 0; b < P.B; ++b) {
    const int64_t Lb = P.seq_off[b + 1] - P.seq_off[b];
    for (int h = 0; h < P.Hkv; ++h) {
      const int64_t kb = p->budgets_h ? p->budgets_h[(size_t)b * P.Hkv + h] : p->k;
      if (kb < 0) return fail(KVSEL_EINVAL, "budgets must be >= 0");
      const int s = b * P.Hkv + h;
      P.keff[s] = (int32_t)std::min<int64_t>(kb, Lb);
      P.out_off[s + 1] = P.out_off[s] + P.keff[s];
    }
  }
  if (p->d != kHeadDim) return fail(KVSEL_EUNSUPPORTED, "this build supports d = 128 only");
  if (P.Hkv > kMaxSeg) return fail(KVSEL_EUNSUPPORTED, "at most 64 KV heads");
  P.R = P.G * P.wp;
  if (P.R > kMaxRows) return fail(KVSEL_EUNSUPPORTED, "at most 512 observation rows (Hq/Hkv * w') per KV head");

  P.has_decode = p->has_decode;
  P.causal = p->causal;
  P.alpha = p->alpha;
  P.pool = p->pool;
  P.pool_kernel = (p->pool == KVSEL_POOL_NONE) ? 1 : p->pool_kernel;
  P.weighting = p->weighting;
  P.sink = p->sink_tokens;
  P.recent = p->recent_tokens;
  if (P.weighting == KVSEL_WEIGHT_EXP) {
    // c_r = exp(lambda r) / sum_r' exp(lambda r') over r = -w+1 .. 0 (.. 1):
    // kept in base 2 and relative to the largest r, so nothing overflows.
    const double lam = p->lambda;
    const int rmax = p->has_decode ? 1 : 0;
    double sum = 0.0;
    for (int j = 0; j < P.w + p->has_decode; ++j) sum += std::exp(lam * (double)(j - (P.w - 1) - rmax));
    P.lam2 = (float)(lam * 1.4426950408889634);
    P.log2norm = (float)std::log2(sum);
  }
  const float scale = (p->scale == 0.0f) ? 1.0f / std::sqrt((float)p->d) : p->scale;
  P.cl2 = (float)((double)scale * 1.4426950408889634);  // log2(e)

  P.nrt = (P.R + kRowTile - 1) / kRowTile;
  P.Rpad = P.nrt * kRowTile;
  const int64_t head_keys = P.seq_off[P.B] * P.Hkv;
  // A caller's key_chunk (TideKV's block size b_s) bounds a block; smaller
  // blocks run the same blockwise procedure with more workgroups.
  P.kb1 = auto_key_block(head_keys, 4096);
  // With one row tile per wave, pass 1 in blocks of twice that size (half
  // as many workgroups): pass 1 itself slows a little, but pass 2 merges
  // half as many block states in its prologue, which gains more (the
  // Llama-shaped 32K layer: 1.96-1.97 against 2.00 ms per 32-layer step);
  // with more row tiles per wave it loses (256 rows per KV head; five row
  // tiles with a decode row).
  if (P.nrt <= kScoreThreads / 64) P.kb1 = std::min(4096, 2 * auto_key_block(head_keys, 2048));
  if (p->key_chunk > 0) P.kb1 = std::min(P.kb1, p->key_chunk);
  // Pass 2 in blocks of at most 2048 keys (its LDS then allows two
  // workgroups per compute unit).  A batch of unequal lengths takes at most
  // 1024 (pass 2) and 2048 (pass 1): the sequences' last, partial blocks
  // leave a launch's last round of workgroups uneven, and finer blocks even
  // it out (a ragged batch of eight 21K-62K sequences: 449-455 against
  // 516-529 us per call; equal lengths and one sequence lose with them).
  bool ragged = false;
  for (int b = 1; b < P.B; ++b)
    ragged |= (P.seq_off[b + 1] - P.seq_off[b]) != (P.seq_off[1] - P.seq_off[0]);
  P.kb2 = auto_key_block(head_keys, ragged ? 1024 : 2048);
  if (ragged) P.kb1 = std::min(P.kb1, 2048);
  P.nblk1_max = (int)((P.Lmax + P.kb1 - 1) / P.kb1);
  P.nblk2_max = (int)((P.Lmax + P.kb2 - 1) / P.kb2);

  const size_t nseg = (size_t)P.B * P.Hkv;
  if (p->stream_keys > 0) return plan_streaming(p, P);
  size_t off = 0;
  P.off_partials = off;
  off = align_up(off + nseg * P.nblk1_max * P.Rpad * sizeof(float2), 256);
  P.off_scores = off;
  off = align_up(off + (size_t)head_keys * sizeof(float), 256);
  P.off_pooled = off;
  off = align_up(off + (size_t)head_keys * sizeof(float), 256);
  P.nchunk_max = (int)((P.Lmax + kSelectChunk - 1) / kSelectChunk);
  const size_t nchunks = nseg * (size_t)P.nchunk_max;
  P.off_tfine = off;
  off = align_up(off + nchunks * kSelectBins * sizeof(uint16_t), 256);
  P.off_tcoarse = off;
  off = align_up(off + nchunks * (kSelectBins / 32) * sizeof(uint16_t), 256);
  P.off_bucket = off;
  off = align_up(off + nchunks * kSelectChunk * sizeof(uint32_t), 256);
  P.off_qmean = off;
  if (P.gqa == KVSEL_GQA_MEAN_QUERY) off = align_up(off + (size_t)P.B * P.wp * P.Hkv * p->d * sizeof(uint16_t), 256);
  // The fused pass 2 of kvsel_compress: pools up to 2 kPoolHalo + 1 wide;
  // its blocks are pass 2's, rounded up to whole table blocks.
  const int pool_r = (P.pool == KVSEL_POOL_NONE) ? 0 : (P.pool_kernel - 1) / 2;
  P.fused = pool_r <= kPoolHalo && !env_unfused();
  if (P.fused) {
    P.kb2t = (P.kb2 + kTabBlock - 1) / kTabBlock * kTabBlock;
    P.ntab_max = (int)((P.Lmax + kTabBlock - 1) / kTabBlock);
    P.off_thist = off;
    off = align_up(off + nseg * kTabHistCopies * kTabBins * sizeof(uint32_t), 256);
    P.off_ttab = off;
    off = align_up(off + nseg * P.ntab_max * kTabBins * sizeof(uint16_t), 256);
    P.off_tbucket = off;
    off = align_up(off + nseg * P.ntab_max * kTabBlock * sizeof(uint32_t), 256);
  }
  P.ws_bytes = off;
  return KVSEL_OK;
}

std::atomic<int> g_device_ok[256];

kvsel_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVSEL_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 256) return fail(KVSEL_EUNSUPPORTED, "device ordinal out of range");
  int st = g_device_ok[dev].load();
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(KVSEL_EHIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_device_ok[dev].store(st);
  }
  if (st != 1) return fail(KVSEL_EUNSUPPORTED, "kernels are built for gfx950 (MI355X) only");
  return KVSEL_OK;
}

kvsel_status check_ptr(const void *ptr, const char *name) {
  if (!ptr) return fail(KVSEL_EINVAL, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0) return fail(KVSEL_EINVAL, std::string(name) + " is not 16-byte aligned");
  return KVSEL_OK;
}

kvsel_status check_ws(const Plan &P, const void *ws, size_t ws_bytes) {
  kvsel_status s = check_ptr(ws, "workspace");
  if (s != KVSEL_OK) return s;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(KVSEL_EINVAL, "workspace is not 256-byte aligned");
  if (ws_bytes < P.ws_bytes)
    return fail(KVSEL_EINVAL, "workspace too small: need " + std::to_string(P.ws_bytes) + " bytes");
  return KVSEL_OK;
}

kvsel_status hip_fail(hipError_t e, const char *what) {
  return fail(KVSEL_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Sequence groups whose segments fit one launch's table.
template <typename F>
kvsel_status for_each_group(const Plan &P, F &&f) {
  const int per = std::max(1, kMaxSeg / P.Hkv);
  for (int s0 = 0; s0 < P.B; s0 += per) {
    SegTable t;
    std::memset(&t, 0, sizeof(t));
    t.nseq = std::min(per, P.B - s0);
    t.seq0 = s0;
    t.seg0 = s0 * P.Hkv;
    int64_t lmax = 0;
    for (int i = 0; i <= t.nseq; ++i) t.key_off[i] = P.seq_off[s0 + i];
    for (int i = 0; i < t.nseq; ++i) lmax = std::max(lmax, t.key_off[i + 1] - t.key_off[i]);
    t.kmax = 0;
    for (int i = 0; i < t.nseq * P.Hkv; ++i) {
      t.keff[i] = P.keff[t.seg0 + i];
      t.out_off[i] = P.out_off[t.seg0 + i];
      t.kmax = std::max(t.kmax, t.keff[i]);
    }
    kvsel_status s = f(t, lmax);
    if (s != KVSEL_OK) return s;
  }
  return KVSEL_OK;
}

ScoreParams score_params(const Plan &P, const void *Q, const void *K, float *scores, char *ws) {
  ScoreParams sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.Q = static_cast<const uint16_t *>(Q);
  if (P.gqa == KVSEL_GQA_MEAN_QUERY) sp.Q = reinterpret_cast<const uint16_t *>(ws + P.off_qmean);
  sp.K = static_cast<const uint16_t *>(K);
  sp.scores = scores;
  sp.partials = reinterpret_cast<float2 *>(ws + P.off_partials);
  sp.Hq = P.Hq;
  sp.Hkv = P.Hkv;
  sp.G = P.G;
  sp.w = P.w;
  sp.wp = P.wp;
  sp.R = P.R;
  sp.Rpad = P.Rpad;
  sp.nrt = P.nrt;
  sp.has_decode = P.has_decode;
  sp.causal = P.causal;
  sp.cl2 = P.cl2;
  sp.alpha = P.alpha;
  sp.weighting = P.weighting;
  sp.lam2 = P.lam2;
  sp.log2norm = P.log2norm;
  sp.nblk1_max = P.nblk1_max;
  sp.stat_block = P.kb1;
  sp.key_begin = 0;
  sp.key_end = INT_MAX;
  sp.out_stride = 0;
  sp.out_origin = 0;
  return sp;
}

// Pass 1: per-block row statistics into the workspace.
// seg_hist (kvsel_compress's fused pass 2): the histograms pass 1 clears.
kvsel_status run_row_stats(const Plan &P, const void *Q, const void *K, char *ws, hipStream_t st,
                           uint32_t *seg_hist = nullptr) {
  if (P.gqa == KVSEL_GQA_MEAN_QUERY) {
    QueryMeanParams qp;
    qp.Q = static_cast<const uint4 *>(Q);
    qp.Qm = reinterpret_cast<uint4 *>(ws + P.off_qmean);
    qp.Hq = P.Hq_in;
    qp.Hkv = P.Hkv;
    qp.G = P.G_in;
    qp.items = P.B * P.wp * P.Hkv;
    hipError_t e = launch_query_mean(qp, st);
    if (e != hipSuccess) return hip_fail(e, "query mean launch");
  }
  ScoreParams sp = score_params(P, Q, K, nullptr, ws);
  sp.seg_hist = seg_hist;
  return for_each_group(P, [&](const SegTable &t, int64_t lmax) {
    sp.key_block = P.kb1;
    hipError_t e = launch_score_pass1(sp, t, (int)((lmax + P.kb1 - 1) / P.kb1), st);
    if (e != hipSuccess) return hip_fail(e, "score pass 1 launch");
    return KVSEL_OK;
  });
}

// Pass 2 (which starts by merging the block statistics into per-row biases).
kvsel_status run_from_stats(const Plan &P, const void *Q, const void *K, float *scores, char *ws, hipStream_t st) {
  ScoreParams sp = score_params(P, Q, K, scores, ws);
  return for_each_group(P, [&](const SegTable &t, int64_t lmax) {
    sp.key_block = P.kb2;
    hipError_t e = launch_score_pass2(sp, t, (int)((lmax + P.kb2 - 1) / P.kb2), st);
    if (e != hipSuccess) return hip_fail(e, "score pass 2 launch");
    return KVSEL_OK;
  });
}

kvsel_status run_score(const Plan &P, const void *Q, const void *K, float *scores, char *ws, hipStream_t st) {
  kvsel_status s = run_row_stats(P, Q, K, ws, st);
  return s == KVSEL_OK ? run_from_stats(P, Q, K, scores, ws, st) : s;
}

// Pool + top-k; with K_out given, also the K/V compaction (fused).
kvsel_status run_select(const Plan &P, const float *scores, float *pooled, int32_t *idx, char *ws, hipStream_t st,
                        const void *K = nullptr, const void *V = nullptr, void *K_out = nullptr,
                        void *V_out = nullptr) {
  SelectParams sp;
  sp.scores = scores;
  sp.pooled = pooled;
  sp.idx = idx;
  sp.tab_fine = reinterpret_cast<uint16_t *>(ws + P.off_tfine);
  sp.tab_coarse = reinterpret_cast<uint16_t *>(ws + P.off_tcoarse);
  sp.bucket = reinterpret_cast<uint32_t *>(ws + P.off_bucket);
  sp.nchunk_max = P.nchunk_max;
  sp.K = static_cast<const uint4 *>(K);
  sp.V = static_cast<const uint4 *>(V);
  sp.K_out = static_cast<uint4 *>(K_out);
  sp.V_out = static_cast<uint4 *>(V_out);
  sp.Hkv = P.Hkv;
  sp.pool = P.pool;
  sp.pool_kernel = P.pool_kernel;
  sp.sink = P.sink;
  sp.recent = P.recent;
  return for_each_group(P, [&](const SegTable &t, int64_t) {
    hipError_t e = launch_pool_topk(sp, t, st);
    if (e != hipSuccess) return hip_fail(e, "pool/top-k launch");
    return KVSEL_OK;
  });
}

kvsel_status run_gather(const Plan &P, const int32_t *idx, const void *K, const void *V, void *Ko, void *Vo,
                        hipStream_t st) {
  GatherParams gp;
  gp.idx = idx;
  gp.K = static_cast<const uint4 *>(K);
  gp.V = static_cast<const uint4 *>(V);
  gp.K_out = static_cast<uint4 *>(Ko);
  gp.V_out = static_cast<uint4 *>(Vo);
  gp.Hkv = P.Hkv;
  return for_each_group(P, [&](const SegTable &t, int64_t) {
    hipError_t e = launch_gather(gp, t, st);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
    return KVSEL_OK;
  });
}

bool any_kept(const Plan &P) { return P.out_off.back() > 0; }


// The pool and reserved positions of pass 2 with the pool, and the sum of
// S over a segment's positions.
void set_pool_params(const Plan &P, ScoreParams &sp) {
  sp.pool = P.pool;
  sp.pool_r = (P.pool == KVSEL_POOL_NONE) ? 0 : (P.pool_kernel - 1) / 2;
  sp.pool_width = (float)P.pool_kernel;
  sp.sink = P.sink;
  sp.recent = P.recent;
  // sum of the row weights: 1 each, or 1 - alpha and alpha with a decode
  // row, or the exponential weights normalised to 1
  double cw = P.w;
  if (P.weighting == KVSEL_WEIGHT_EXP) cw = 1.0;
  else if (P.has_decode) cw = (1.0 - P.alpha) * P.w + P.alpha;
  sp.wsum = (float)(P.G * cw);
}

kvsel_status run_compress_fused(const Plan &P, const void *Q, const void *K, const void *V, int32_t *idx, void *K_out,
                                void *V_out, float *pooled, char *ws, hipStream_t st) {
  uint32_t *seg_hist = reinterpret_cast<uint32_t *>(ws + P.off_thist);
  kvsel_status s = run_row_stats(P, Q, K, ws, st, seg_hist);
  if (s != KVSEL_OK) return s;
  ScoreParams sp = score_params(P, Q, K, nullptr, ws);
  sp.pooled = pooled;
  sp.tab = reinterpret_cast<uint16_t *>(ws + P.off_ttab);
  sp.bucket = reinterpret_cast<uint32_t *>(ws + P.off_tbucket);
  sp.seg_hist = seg_hist;
  sp.ntab_max = P.ntab_max;
  set_pool_params(P, sp);

  SelectParams sel;
  std::memset(&sel, 0, sizeof(sel));
  sel.pooled = pooled;
  sel.idx = idx;
  sel.tab_fine = sp.tab;
  sel.bucket = sp.bucket;
  sel.seg_hist = sp.seg_hist;
  sel.nblk_max = P.ntab_max;
  sel.Hkv = P.Hkv;
  sel.pool = P.pool;
  sel.pool_kernel = P.pool_kernel;
  sel.sink = P.sink;
  sel.recent = P.recent;
  if (any_kept(P)) {
    sel.K = static_cast<const uint4 *>(K);
    sel.V = static_cast<const uint4 *>(V);
    sel.K_out = static_cast<uint4 *>(K_out);
    sel.V_out = static_cast<uint4 *>(V_out);
  }
  return for_each_group(P, [&](const SegTable &t, int64_t lmax) {
    sp.key_block = P.kb2t;
    hipError_t e = launch_score_pass2_tables(sp, t, (int)((lmax + P.kb2t - 1) / P.kb2t), st);
    if (e != hipSuccess) return hip_fail(e, "score pass 2 launch");
    if (t.kmax > 0) {  // some segment of the group keeps a row
      e = launch_select_blocks(sel, t, st);
      if (e != hipSuccess) return hip_fail(e, "selection launch");
    }
    return KVSEL_OK;
  });
}

}  // namespace

namespace {

// TideKV §4.2's streaming form of steps 1-7 with a workspace bounded by the
// keys per step: pass 1 step by step into running row states, the merge
// into biases, then pass 2 step by step, each step's pooled scores merged
// into the running top-k by the exact selection kernels, and the gather.
kvsel_status run_compress_streaming(const Plan &P, const void *Q, const void *K, const void *V, int32_t *idx,
                                    void *K_out, void *V_out, char *ws, hipStream_t st) {
  if (P.gqa == KVSEL_GQA_MEAN_QUERY) {
    QueryMeanParams qp;
    qp.Q = static_cast<const uint4 *>(Q);
    qp.Qm = reinterpret_cast<uint4 *>(ws + P.off_qmean);
    qp.Hq = P.Hq_in;
    qp.Hkv = P.Hkv;
    qp.G = P.G_in;
    qp.items = P.B * P.wp * P.Hkv;
    hipError_t e = launch_query_mean(qp, st);
    if (e != hipSuccess) return hip_fail(e, "query mean launch");
  }
  const int nsteps = (int)((P.Lmax + P.stream - 1) / P.stream);
  float2 *run = reinterpret_cast<float2 *>(ws + P.off_run);
  ScoreParams sp = score_params(P, Q, K, nullptr, ws);
  kvsel_status s = KVSEL_OK;
  // Pass 1, step by step.
  for (int c = 0; c < nsteps && s == KVSEL_OK; ++c) {
    const int c0 = c * P.stream;
    sp.key_block = P.kb1;
    sp.key_begin = c0;
    sp.key_end = c0 + P.stream;
    s = for_each_group(P, [&](const SegTable &t, int64_t lmax) {
      if (c0 < lmax) {
        const int nblk = (int)((std::min<int64_t>(lmax, c0 + P.stream) - c0 + P.kb1 - 1) / P.kb1);
        hipError_t e = launch_score_pass1(sp, t, nblk, st);
        if (e != hipSuccess) return hip_fail(e, "score pass 1 launch");
      }
      hipError_t e = launch_stream_stats(sp, t, run, c == 0, st);
      if (e != hipSuccess) return hip_fail(e, "row statistics fold launch");
      return KVSEL_OK;
    });
  }
  if (s != KVSEL_OK) return s;
  // Pass 2 takes its biases from the running states: one block state per
  // row and segment.
  sp.partials = run;
  sp.nblk1_max = 1;
  sp.stat_block = 1 << 30;
  // Pass 2 and the running selection, step by step.
  StreamParams q;
  q.S = reinterpret_cast<const float *>(ws + P.off_sbuf);
  q.S_stride = (int64_t)P.stream + 2 * P.halo;
  q.lv = P.lv;
  q.kslot = P.kslot;
  q.stream = P.stream;
  q.Hkv = P.Hkv;
  q.pool = P.pool;
  q.pool_kernel = P.pool_kernel;
  q.sink = P.sink;
  q.recent = P.recent;
  q.sel = reinterpret_cast<const int32_t *>(ws + P.off_selidx);
  int cur = 0;
  q.cand = reinterpret_cast<float *>(ws + P.off_cand[cur]);
  s = for_each_group(P, [&](const SegTable &t, int64_t) {
    hipError_t e = launch_stream_init(q, t, st);
    if (e != hipSuccess) return hip_fail(e, "streaming init launch");
    return KVSEL_OK;
  });
  if (s != KVSEL_OK) return s;
  sp.scores = reinterpret_cast<float *>(ws + P.off_sbuf);
  sp.out_stride = q.S_stride;
  for (int c = 0; c < nsteps; ++c) {
    const int c0 = c * P.stream;
    sp.key_block = P.kb2;
    sp.key_begin = std::max(0, c0 - P.halo);
    sp.key_end = c0 + P.stream + P.halo;
    sp.out_origin = c0 - P.halo;
    q.c0 = c0;
    q.S_origin = c0 - P.halo;
    q.cand = reinterpret_cast<float *>(ws + P.off_cand[cur]);
    q.cand_next = reinterpret_cast<float *>(ws + P.off_cand[cur ^ 1]);
    q.pos_in = reinterpret_cast<const int32_t *>(ws + P.off_pos[cur]);
    q.pos_out = reinterpret_cast<int32_t *>(ws + P.off_pos[cur ^ 1]);
    s = for_each_group(P, [&](const SegTable &t, int64_t lmax) {
      if (sp.key_begin < lmax) {
        const int64_t hi = std::min<int64_t>(lmax, sp.key_end);
        const int nblk = (int)((hi - sp.key_begin + P.kb2 - 1) / P.kb2);
        hipError_t e = launch_score_pass2(sp, t, nblk, st);
        if (e != hipSuccess) return hip_fail(e, "score pass 2 launch");
      }
      hipError_t e = launch_stream_pool(q, t, st);
      if (e != hipSuccess) return hip_fail(e, "streaming pool launch");
      return KVSEL_OK;
    });
    if (s != KVSEL_OK) return s;
    // The step's selection: one candidate row per segment, budget
    // min(k, keys seen so far), no pool (the row holds pooled values), no
    // reserve (reserved positions carry +inf).
    Plan V = P;
    V.pool = KVSEL_POOL_NONE;
    V.pool_kernel = 1;
    V.sink = 0;
    V.recent = 0;
    V.Lmax = P.lv;
    for (int b = 0; b <= P.B; ++b) V.seq_off[b] = (int64_t)b * P.lv;
    for (int b = 0; b < P.B; ++b) {
      const int64_t seen = std::min<int64_t>(P.seq_off[b + 1] - P.seq_off[b], (int64_t)c0 + P.stream);
      for (int h = 0; h < P.Hkv; ++h) {
        const size_t sg = (size_t)b * P.Hkv + h;
        V.keff[sg] = (int32_t)std::min<int64_t>(P.keff[sg], seen);
        V.out_off[sg + 1] = V.out_off[sg] + V.keff[sg];
      }
    }
    if (any_kept(V)) {
      s = run_select(V, q.cand, reinterpret_cast<float *>(ws + P.off_candp), reinterpret_cast<int32_t *>(ws + P.off_selidx),
                     ws, st);
      if (s != KVSEL_OK) return s;
    }
    s = for_each_group(V, [&](const SegTable &vt, int64_t) {
      hipError_t e = launch_stream_map(q, vt, st);
      if (e != hipSuccess) return hip_fail(e, "streaming map launch");
      return KVSEL_OK;
    });
    if (s != KVSEL_OK) return s;
    cur ^= 1;
  }
  q.pos_in = reinterpret_cast<const int32_t *>(ws + P.off_pos[cur]);
  s = for_each_group(P, [&](const SegTable &t, int64_t) {
    hipError_t e = launch_stream_final(q, t, idx, st);
    if (e != hipSuccess) return hip_fail(e, "streaming result launch");
    return KVSEL_OK;
  });
  if (s != KVSEL_OK) return s;
  return any_kept(P) ? run_gather(P, idx, K, V, K_out, V_out, st) : KVSEL_OK;
}

// The fused streaming form: pass 1 once over the whole prefix; then per
// step of C keys, pass 2 with the pool writes the step's order keys behind
// the running ones and one selection launch keeps the best keff of each
// row; the last step's selection writes idx, and the gather follows.
kvsel_status run_compress_stream_fused(const Plan &P, const void *Q, const void *K, const void *V, int32_t *idx,
                                       void *K_out, void *V_out, char *ws, hipStream_t st) {
  kvsel_status s = run_row_stats(P, Q, K, ws, st);  // (and the mean queries)
  if (s != KVSEL_OK) return s;
  ScoreParams sp = score_params(P, Q, K, nullptr, ws);
  // The block states merged once into one state per row, which every step's
  // pass 2 then takes as its only block state.
  float2 *run = reinterpret_cast<float2 *>(ws + P.off_run);
  sp.key_block = P.kb1;
  s = for_each_group(P, [&](const SegTable &t, int64_t) {
    hipError_t e = launch_stream_stats(sp, t, run, 1, st);
    if (e != hipSuccess) return hip_fail(e, "row statistics merge launch");
    return KVSEL_OK;
  });
  if (s != KVSEL_OK) return s;
  sp.partials = run;
  sp.nblk1_max = 1;
  sp.stat_block = 1 << 30;
  set_pool_params(P, sp);
  sp.step_stride = P.lv;
  sp.key_block = P.kb2s;
  uint32_t *keys[2];
  int32_t *pos[2];
  for (int i = 0; i < 2; ++i) {
    keys[i] = reinterpret_cast<uint32_t *>(ws + P.off_skeys[i]);
    pos[i] = reinterpret_cast<int32_t *>(ws + P.off_spos[i]);
  }
  StreamSelectParams q;
  std::memset(&q, 0, sizeof(q));
  q.idx = idx;
  q.lv = P.lv;
  q.kslot = P.kslot;
  q.stream = P.stream;
  q.Hkv = P.Hkv;
  q.wsum = sp.wsum;
  s = for_each_group(P, [&](const SegTable &t, int64_t lmax) {
    const int nsteps = (int)((lmax + P.stream - 1) / P.stream);
    for (int c = 0; c < nsteps; ++c) {
      const int c0 = c * P.stream;
      sp.key_begin = c0;
      sp.key_end = c0 + P.stream;
      sp.step_keys = keys[c & 1] + P.kslot;
      sp.step_origin = c0;
      const int64_t hi = std::min<int64_t>(lmax, (int64_t)c0 + P.stream);
      hipError_t e = launch_score_pass2_keys(sp, t, (int)((hi - c0 + P.kb2s - 1) / P.kb2s), st);
      if (e != hipSuccess) return hip_fail(e, "score pass 2 launch");
      if (t.kmax <= 0) continue;  // no segment of the group keeps a row
      q.keys_in = keys[c & 1];
      q.pos_in = pos[c & 1];
      q.keys_out = keys[(c + 1) & 1];
      q.pos_out = pos[(c + 1) & 1];
      q.c0 = c0;
      q.last = (c == nsteps - 1) ? 1 : 0;
      e = launch_stream_select(q, t, st);
      if (e != hipSuccess) return hip_fail(e, "streaming selection launch");
    }
    return KVSEL_OK;
  });
  if (s != KVSEL_OK) return s;
  return any_kept(P) ? run_gather(P, idx, K, V, K_out, V_out, st) : KVSEL_OK;
}

kvsel_status reject_streaming(const Plan &P, const char *fn) {
  if (P.stream > 0)
    return fail(KVSEL_EINVAL, std::string(fn) + " needs whole-prefix buffers; stream_keys applies to kvsel_compress only");
  return KVSEL_OK;
}

}  // namespace

kvsel_status kvsel::set_error(kvsel_status s, const char *msg) { return fail(s, msg); }

KVSEL_API int kvsel_abi_version(void) { return KVSEL_ABI_VERSION; }

KVSEL_API const char *kvsel_status_string(kvsel_status s) {
  switch (s) {
    case KVSEL_OK: return "ok";
    case KVSEL_EINVAL: return "invalid argument";
    case KVSEL_EUNSUPPORTED: return "unsupported";
    case KVSEL_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

KVSEL_API const char *kvsel_last_error(void) { return g_last_error.c_str(); }

KVSEL_API kvsel_status kvsel_plan(const kvsel_problem *p, size_t *workspace_bytes, int64_t *out_offsets_h) {
  g_last_error.clear();
  if (!workspace_bytes) return fail(KVSEL_EINVAL, "workspace_bytes is NULL");
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s != KVSEL_OK) return s;
  *workspace_bytes = P.ws_bytes;
  if (out_offsets_h) std::memcpy(out_offsets_h, P.out_off.data(), P.out_off.size() * sizeof(int64_t));
  return KVSEL_OK;
}

KVSEL_API kvsel_status kvsel_score(const kvsel_problem *p, const void *Q, const void *K, float *scores, void *ws,
                                   size_t ws_bytes, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = reject_streaming(P, "kvsel_score");
  if (s == KVSEL_OK) s = check_ptr(Q, "Q");
  if (s == KVSEL_OK) s = check_ptr(K, "K");
  if (s == KVSEL_OK) s = check_ptr(scores, "scores");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  return run_score(P, Q, K, scores, static_cast<char *>(ws), reinterpret_cast<hipStream_t>(stream));
}

KVSEL_API kvsel_status kvsel_row_stats(const kvsel_problem *p, const void *Q, const void *K, void *ws,
                                       size_t ws_bytes, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = reject_streaming(P, "kvsel_row_stats");
  if (s == KVSEL_OK) s = check_ptr(Q, "Q");
  if (s == KVSEL_OK) s = check_ptr(K, "K");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  return run_row_stats(P, Q, K, static_cast<char *>(ws), reinterpret_cast<hipStream_t>(stream));
}

KVSEL_API kvsel_status kvsel_score_from_stats(const kvsel_problem *p, const void *Q, const void *K, float *scores,
                                              void *ws, size_t ws_bytes, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = reject_streaming(P, "kvsel_score_from_stats");
  if (s == KVSEL_OK) s = check_ptr(Q, "Q");
  if (s == KVSEL_OK) s = check_ptr(K, "K");
  if (s == KVSEL_OK) s = check_ptr(scores, "scores");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  return run_from_stats(P, Q, K, scores, static_cast<char *>(ws), reinterpret_cast<hipStream_t>(stream));
}

KVSEL_API kvsel_status kvsel_pool_topk(const kvsel_problem *p, const float *scores, float *pooled, int32_t *idx,
                                       void *ws, size_t ws_bytes, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = reject_streaming(P, "kvsel_pool_topk");
  if (s == KVSEL_OK) s = check_ptr(scores, "scores");
  if (s == KVSEL_OK && pooled) s = check_ptr(pooled, "pooled");
  if (s == KVSEL_OK && any_kept(P)) s = check_ptr(idx, "idx");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  float *pool_buf = pooled ? pooled : reinterpret_cast<float *>(static_cast<char *>(ws) + P.off_pooled);
  return run_select(P, scores, pool_buf, idx, static_cast<char *>(ws), reinterpret_cast<hipStream_t>(stream));
}

KVSEL_API kvsel_status kvsel_gather(const kvsel_problem *p, const int32_t *idx, const void *K, const void *V,
                                    void *K_out, void *V_out, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = check_ptr(K, "K");
  if (s == KVSEL_OK) s = check_ptr(V, "V");
  if (s == KVSEL_OK && any_kept(P)) s = check_ptr(idx, "idx");
  if (s == KVSEL_OK && any_kept(P)) s = check_ptr(K_out, "K_out");
  if (s == KVSEL_OK && any_kept(P)) s = check_ptr(V_out, "V_out");
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  if (!any_kept(P)) return KVSEL_OK;
  return run_gather(P, idx, K, V, K_out, V_out, reinterpret_cast<hipStream_t>(stream));
}


KVSEL_API kvsel_status kvsel_compress(const kvsel_problem *p, const void *Q, const void *K, const void *V,
                                      int32_t *idx, void *K_out, void *V_out, float *pooled, void *ws,
                                      size_t ws_bytes, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = check_ptr(Q, "Q");
  if (s == KVSEL_OK) s = check_ptr(K, "K");
  if (s == KVSEL_OK) s = check_ptr(V, "V");
  if (s == KVSEL_OK && any_kept(P)) s = check_ptr(idx, "idx");
  if (s == KVSEL_OK && any_kept(P)) s = check_ptr(K_out, "K_out");
  if (s == KVSEL_OK && any_kept(P)) s = check_ptr(V_out, "V_out");
  if (s == KVSEL_OK && pooled) s = check_ptr(pooled, "pooled");
  if (s == KVSEL_OK && pooled && P.stream > 0)
    s = fail(KVSEL_EINVAL, "pooled must be NULL with stream_keys (no whole-prefix pooled scores are kept)");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  char *wsb = static_cast<char *>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (P.stream > 0 && P.sfused) return run_compress_stream_fused(P, Q, K, V, idx, K_out, V_out, wsb, st);
  if (P.stream > 0) return run_compress_streaming(P, Q, K, V, idx, K_out, V_out, wsb, st);
  float *scores = reinterpret_cast<float *>(wsb + P.off_scores);
  float *pool_buf = pooled ? pooled : reinterpret_cast<float *>(wsb + P.off_pooled);
  if (P.fused) return run_compress_fused(P, Q, K, V, idx, K_out, V_out, pool_buf, wsb, st);
  s = run_score(P, Q, K, scores, wsb, st);
  if (s != KVSEL_OK) return s;
  if (any_kept(P)) return run_select(P, scores, pool_buf, idx, wsb, st, K, V, K_out, V_out);
  return run_select(P, scores, pool_buf, idx, wsb, st);
}

namespace {

// The ranking of a warm-up profile as a selection problem: one segment per
// sequence (a single "head"), budget min(n, L_b), no reserved positions.
Plan tier_plan(const Plan &P, int64_t n) {
  Plan V = P;
  V.Hkv = 1;
  V.sink = 0;
  V.recent = 0;
  V.keff.assign((size_t)P.B, 0);
  V.out_off.assign((size_t)P.B + 1, 0);
  for (int b = 0; b < P.B; ++b) {
    const int64_t Lb = P.seq_off[b + 1] - P.seq_off[b];
    V.keff[b] = (int32_t)std::min<int64_t>(n, Lb);
    V.out_off[b + 1] = V.out_off[b] + V.keff[b];
  }
  return V;
}

}  // namespace

KVSEL_API kvsel_status kvsel_profile_layer(const kvsel_problem *p, const void *Q, const void *K, float *profile,
                                           int32_t accumulate, void *ws, size_t ws_bytes, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = reject_streaming(P, "kvsel_profile_layer");
  if (s == KVSEL_OK) s = check_ptr(Q, "Q");
  if (s == KVSEL_OK) s = check_ptr(K, "K");
  if (s == KVSEL_OK) s = check_ptr(profile, "profile");
  if (s == KVSEL_OK && accumulate != 0 && accumulate != 1) s = fail(KVSEL_EINVAL, "accumulate must be 0 or 1");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  char *wsb = static_cast<char *>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float *scores = reinterpret_cast<float *>(wsb + P.off_scores);
  s = run_score(P, Q, K, scores, wsb, st);
  if (s != KVSEL_OK) return s;
  ProfileParams pp;
  pp.scores = scores;
  pp.profile = profile;
  pp.Hkv = P.Hkv;
  pp.accumulate = accumulate;
  return for_each_group(P, [&](const SegTable &t, int64_t lmax) {
    hipError_t e = launch_profile(pp, t, lmax, st);
    if (e != hipSuccess) return hip_fail(e, "profile launch");
    return KVSEL_OK;
  });
}

KVSEL_API kvsel_status kvsel_tier_rank(const kvsel_problem *p, const float *profile, int64_t n_fast, int64_t n_mid,
                                       int8_t *tier, void *ws, size_t ws_bytes, kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = reject_streaming(P, "kvsel_tier_rank");
  if (s == KVSEL_OK) s = check_ptr(profile, "profile");
  if (s == KVSEL_OK) s = check_ptr(tier, "tier");
  if (s == KVSEL_OK && (n_fast < 0 || n_mid < 0)) s = fail(KVSEL_EINVAL, "n_fast and n_mid must be >= 0");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  char *wsb = static_cast<char *>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // The selection's positions go where the per-head scores would live; the
  // pooled profile where the pooled scores would.  Both regions hold at
  // least sum L_b four-byte values.
  int32_t *idx = reinterpret_cast<int32_t *>(wsb + P.off_scores);
  float *pooled = reinterpret_cast<float *>(wsb + P.off_pooled);
  hipError_t e = launch_tier_fill(tier, P.seq_off[P.B], st);
  if (e != hipSuccess) return hip_fail(e, "tier fill launch");
  const int64_t cap = P.Lmax;  // a budget beyond the longest sequence keeps everything
  const int64_t ranks[2] = {std::min(cap, n_fast) + std::min(cap, n_mid), std::min(cap, n_fast)};
  for (int pass = 0; pass < 2; ++pass) {
    const Plan V = tier_plan(P, ranks[pass]);
    if (!any_kept(V)) continue;
    s = run_select(V, profile, pooled, idx, wsb, st);
    if (s != KVSEL_OK) return s;
    const int label = 1 - pass;  // the middle tier's selection first, then the fast tier's
    s = for_each_group(V, [&](const SegTable &t, int64_t) {
      hipError_t e2 = launch_tier_mark(idx, tier, label, t, st);
      if (e2 != hipSuccess) return hip_fail(e2, "tier mark launch");
      return KVSEL_OK;
    });
    if (s != KVSEL_OK) return s;
  }
  return KVSEL_OK;
}

KVSEL_API kvsel_status kvsel_topk_mass(const kvsel_problem *p, const float *pooled, int32_t n_sizes,
                                       const int32_t *sizes_h, float *mass, void *ws, size_t ws_bytes,
                                       kvsel_stream_t stream) {
  g_last_error.clear();
  Plan P;
  kvsel_status s = make_plan(p, P);
  if (s == KVSEL_OK) s = reject_streaming(P, "kvsel_topk_mass");
  if (s == KVSEL_OK) s = check_ptr(pooled, "pooled");
  if (s == KVSEL_OK) s = check_ptr(mass, "mass");
  if (s == KVSEL_OK && (n_sizes < 1 || !sizes_h)) s = fail(KVSEL_EINVAL, "need n_sizes >= 1 candidate sizes");
  for (int j = 0; s == KVSEL_OK && j < n_sizes; ++j)
    if (sizes_h[j] < 0) s = fail(KVSEL_EINVAL, "sizes must be >= 0");
  if (s == KVSEL_OK) s = check_ws(P, ws, ws_bytes);
  if (s == KVSEL_OK) s = check_device();
  if (s != KVSEL_OK) return s;
  char *wsb = static_cast<char *>(ws);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // Kept positions where the unpooled scores would live (at most sum L_b * Hkv).
  int32_t *idx = reinterpret_cast<int32_t *>(wsb + P.off_scores);
  float *copy = reinterpret_cast<float *>(wsb + P.off_pooled);
  for (int j = 0; j < n_sizes; ++j) {
    // The given pooled scores, unpooled again, with the uniform budget
    // sizes_h[j] and no reserved positions.
    Plan V = P;
    V.pool = KVSEL_POOL_NONE;
    V.pool_kernel = 1;
    V.sink = 0;
    V.recent = 0;
    for (int b = 0; b < P.B; ++b) {
      const int64_t Lb = P.seq_off[b + 1] - P.seq_off[b];
      for (int h = 0; h < P.Hkv; ++h) {
        const size_t sg = (size_t)b * P.Hkv + h;
        V.keff[sg] = (int32_t)std::min<int64_t>(sizes_h[j], Lb);
        V.out_off[sg + 1] = V.out_off[sg] + V.keff[sg];
      }
    }
    s = run_select(V, pooled, copy, idx, wsb, st);
    if (s != KVSEL_OK) return s;
    MassParams mp;
    mp.pooled = pooled;
    mp.idx = idx;
    mp.mass = mass;
    mp.Hkv = P.Hkv;
    mp.n_sizes = n_sizes;
    mp.j = j;
    s = for_each_group(V, [&](const SegTable &t, int64_t) {
      hipError_t e = launch_mass(mp, t, st);
      if (e != hipSuccess) return hip_fail(e, "mass launch");
      return KVSEL_OK;
    });
    if (s != KVSEL_OK) return s;
  }
  return KVSEL_OK;
}

KVSEL_API kvsel_status kvsel_allocate_budgets(int32_t n_items, int32_t n_sizes, const int32_t *sizes_h,
                                              const double *benefit_h, int64_t total, int32_t *budgets_h) {
  g_last_error.clear();
  if (n_items < 0 || n_sizes < 1) return fail(KVSEL_EINVAL, "need n_items >= 0 and n_sizes >= 1");
  if (n_items == 0) return KVSEL_OK;
  if (!sizes_h || !benefit_h || !budgets_h) return fail(KVSEL_EINVAL, "NULL argument");
  for (int j = 0; j < n_sizes; ++j) {
    if (sizes_h[j] < 0) return fail(KVSEL_EINVAL, "sizes must be >= 0");
    if (j > 0 && sizes_h[j] <= sizes_h[j - 1]) return fail(KVSEL_EINVAL, "sizes must be strictly increasing");
  }
  for (int64_t i = 0; i < (int64_t)n_items * n_sizes; ++i)
    if (!std::isfinite(benefit_h[i])) return fail(KVSEL_EINVAL, "benefits must be finite");
  // Every pair starts at the smallest size; then the step with the largest
  // added benefit per added entry among those that fit is taken, lowest pair
  // first on equal ratios, until no step fits or adds benefit.
  std::vector<int> choice((size_t)n_items, 0);
  int64_t left = total - (int64_t)n_items * sizes_h[0];
  if (left >= 0) {
    for (;;) {
      int best = -1;
      double best_ratio = 0.0;
      for (int i = 0; i < n_items; ++i) {
        const int j = choice[i];
        if (j + 1 >= n_sizes) continue;
        const int64_t dc = (int64_t)sizes_h[j + 1] - sizes_h[j];
        const double db = benefit_h[(int64_t)i * n_sizes + j + 1] - benefit_h[(int64_t)i * n_sizes + j];
        if (dc > left || !(db > 0.0)) continue;
        const double ratio = db / (double)dc;
        if (ratio > best_ratio) {
          best = i;
          best_ratio = ratio;
        }
      }
      if (best < 0) break;
      left -= (int64_t)sizes_h[choice[best] + 1] - sizes_h[choice[best]];
      ++choice[best];
    }
  }
  for (int i = 0; i < n_items; ++i) budgets_h[i] = sizes_h[choice[i]];
  return KVSEL_OK;
}
