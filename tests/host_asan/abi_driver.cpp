// The host library (kvsel_api.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer against the stand-in launches of
// launch_stubs.cpp, driven through every entry point of include/kvsel.h:
// invalid problems and arguments must be rejected without touching memory
// out of bounds, and valid ones must plan and launch with every kernel
// array inside the caller's buffers.  Exits 0 when every check passes.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kvsel.h"
#include "registry.h"

namespace {

int g_fail = 0;

void check(bool ok, const std::string &what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL %s\n", what.c_str());
    ++g_fail;
  }
}

kvsel_problem base_problem() {
  kvsel_problem p;
  std::memset(&p, 0, sizeof(p));
  p.batch = 1;
  p.Hq = 32;
  p.Hkv = 8;
  p.d = 128;
  p.L = 4096;
  p.w = 32;
  p.causal = 1;
  p.pool = KVSEL_POOL_MAX;
  p.pool_kernel = 7;
  p.k = 512;
  return p;
}

// A buffer of n bytes (256-byte aligned, never read or written here),
// registered for the stand-in launches.
struct Arena {
  std::vector<void *> ptrs;
  void *get(size_t n, const char *name) {
    const size_t sz = (n + 255) / 256 * 256 + 256;
    void *p = std::aligned_alloc(256, sz);
    ptrs.push_back(p);
    reg_add(p, n, name);
    return p;
  }
  ~Arena() {
    for (void *p : ptrs) std::free(p);
    reg_clear();
  }
};

struct Shape {
  std::string name;
  kvsel_problem p;
  std::vector<int64_t> offs;   // seq offsets (empty: uniform L)
  std::vector<int32_t> budgets;
};

void run_shape(Shape &s) {
  kvsel_problem &p = s.p;
  if (!s.offs.empty()) p.seq_offsets_h = s.offs.data();
  if (!s.budgets.empty()) p.budgets_h = s.budgets.data();
  size_t ws = 0;
  const int64_t nseg = (int64_t)p.batch * p.Hkv;
  std::vector<int64_t> out_off(nseg + 1);
  kvsel_status st = kvsel_plan(&p, &ws, out_off.data());
  check(st == KVSEL_OK, s.name + ": plan: " + kvsel_last_error());
  if (st != KVSEL_OK) return;
  const int64_t keys = s.offs.empty() ? p.L * p.batch : s.offs.back();
  const int64_t kept = out_off[nseg];
  const int64_t wp = p.w + p.has_decode;
  Arena a;
  void *Q = a.get((size_t)p.batch * wp * p.Hq * p.d * 2, "Q");
  void *K = a.get((size_t)keys * p.Hkv * p.d * 2, "K");
  void *V = a.get((size_t)keys * p.Hkv * p.d * 2, "V");
  float *scores = static_cast<float *>(a.get((size_t)keys * p.Hkv * 4, "scores"));
  float *pooled = static_cast<float *>(a.get((size_t)keys * p.Hkv * 4, "pooled"));
  int32_t *idx = static_cast<int32_t *>(a.get((size_t)std::max<int64_t>(kept, 1) * 4, "idx"));
  void *Ko = a.get((size_t)std::max<int64_t>(kept, 1) * p.d * 2, "K_out");
  void *Vo = a.get((size_t)std::max<int64_t>(kept, 1) * p.d * 2, "V_out");
  void *W = a.get(ws, "workspace");
  float *profile = static_cast<float *>(a.get((size_t)keys * 4, "profile"));
  int8_t *tier = static_cast<int8_t *>(a.get((size_t)keys, "tier"));
  const int32_t sizes[3] = {16, 64, 256};
  float *mass = static_cast<float *>(a.get((size_t)nseg * 3 * 4, "mass"));
  auto ok = [&](kvsel_status r, const char *what) {
    check(r == KVSEL_OK, s.name + ": " + what + ": " + kvsel_status_string(r) + " " + kvsel_last_error());
  };
  if (p.stream_keys > 0) {
    ok(kvsel_compress(&p, Q, K, V, idx, Ko, Vo, nullptr, W, ws, nullptr), "streaming compress");
    check(kvsel_score(&p, Q, K, scores, W, ws, nullptr) == KVSEL_EINVAL, s.name + ": score rejects streaming");
    return;
  }
  ok(kvsel_score(&p, Q, K, scores, W, ws, nullptr), "score");
  ok(kvsel_row_stats(&p, Q, K, W, ws, nullptr), "row stats");
  ok(kvsel_score_from_stats(&p, Q, K, scores, W, ws, nullptr), "score from stats");
  ok(kvsel_pool_topk(&p, scores, pooled, idx, W, ws, nullptr), "pool/top-k");
  ok(kvsel_gather(&p, idx, K, V, Ko, Vo, nullptr), "gather");
  ok(kvsel_compress(&p, Q, K, V, idx, Ko, Vo, pooled, W, ws, nullptr), "compress");
  ok(kvsel_compress(&p, Q, K, V, idx, Ko, Vo, nullptr, W, ws, nullptr), "compress without pooled");
  setenv("KVSEL_UNFUSED", "1", 1);
  ok(kvsel_compress(&p, Q, K, V, idx, Ko, Vo, pooled, W, ws, nullptr), "compress, unfused");
  unsetenv("KVSEL_UNFUSED");
  ok(kvsel_profile_layer(&p, Q, K, profile, 0, W, ws, nullptr), "profile");
  ok(kvsel_tier_rank(&p, profile, 100, 300, tier, W, ws, nullptr), "tier rank");
  ok(kvsel_topk_mass(&p, pooled, 3, sizes, mass, W, ws, nullptr), "top-k mass");
  // argument errors: too small a workspace, misaligned and NULL pointers
  check(kvsel_compress(&p, Q, K, V, idx, Ko, Vo, pooled, W, ws - 1, nullptr) == KVSEL_EINVAL,
        s.name + ": small workspace rejected");
  check(kvsel_score(&p, static_cast<char *>(Q) + 4, K, scores, W, ws, nullptr) == KVSEL_EINVAL,
        s.name + ": misaligned Q rejected");
  check(kvsel_score(&p, Q, nullptr, scores, W, ws, nullptr) == KVSEL_EINVAL, s.name + ": NULL K rejected");
}

}  // namespace

int main() {
  // ---- invalid problems: rejected by the planner, nothing else happens
  {
    std::vector<std::pair<std::string, kvsel_problem>> bad;
    auto add = [&](const char *n, void (*f)(kvsel_problem &)) {
      kvsel_problem p = base_problem();
      f(p);
      bad.push_back({n, p});
    };
    add("d 64", [](kvsel_problem &p) { p.d = 64; });
    add("Hq not a multiple", [](kvsel_problem &p) { p.Hq = 30; });
    add("Hkv 0", [](kvsel_problem &p) { p.Hkv = 0; });
    add("w 0", [](kvsel_problem &p) { p.w = 0; });
    add("w past L", [](kvsel_problem &p) { p.L = 8; p.w = 9; });
    add("even pool", [](kvsel_problem &p) { p.pool_kernel = 4; });
    add("pool kernel 257", [](kvsel_problem &p) { p.pool_kernel = 257; });
    add("k negative", [](kvsel_problem &p) { p.k = -1; });
    add("alpha 2", [](kvsel_problem &p) { p.has_decode = 1; p.alpha = 2.0f; });
    add("key chunk 48", [](kvsel_problem &p) { p.key_chunk = 48; });
    add("scale inf", [](kvsel_problem &p) { p.scale = 1.0f / 0.0f; });
    add("weighting 2", [](kvsel_problem &p) { p.weighting = 2; });
    add("lambda negative", [](kvsel_problem &p) { p.weighting = 1; p.lambda = -1.0f; });
    add("gqa 2", [](kvsel_problem &p) { p.gqa = 2; });
    add("stream 1000", [](kvsel_problem &p) { p.stream_keys = 1000; });
    add("L 2^20 + 1", [](kvsel_problem &p) { p.L = (1 << 20) + 1; });
    add("batch 0", [](kvsel_problem &p) { p.batch = 0; });
    for (auto &b : bad) {
      size_t ws = 0;
      std::vector<int64_t> offs(1024);
      const kvsel_status st = kvsel_plan(&b.second, &ws, offs.data());
      check(st == KVSEL_EINVAL || st == KVSEL_EUNSUPPORTED, "bad problem accepted: " + b.first);
    }
    check(kvsel_plan(nullptr, nullptr, nullptr) == KVSEL_EINVAL, "NULL problem");
  }

  // ---- valid problems through every entry point
  std::vector<Shape> shapes;
  {
    Shape s{"c1 4096", base_problem(), {}, {}};
    s.p.pool = KVSEL_POOL_AVG;
    shapes.push_back(s);
  }
  {
    Shape s{"c2 32768", base_problem(), {}, {}};
    s.p.L = 32768;
    s.p.k = 2048;
    shapes.push_back(s);
  }
  {
    Shape s{"c3-like 131072 w64 chunk 4096", base_problem(), {}, {}};
    s.p.L = 131072;
    s.p.w = 64;
    s.p.key_chunk = 4096;
    s.p.k = 4096;
    shapes.push_back(s);
  }
  {
    Shape s{"c4-like B4 decode", base_problem(), {}, {}};
    s.p.batch = 4;
    s.p.L = 65536;
    s.p.has_decode = 1;
    s.p.alpha = 0.5f;
    s.p.pool_kernel = 5;
    s.p.k = 2048;
    shapes.push_back(s);
  }
  {
    Shape s{"ragged budgets", base_problem(), {0, 300, 377, 1408}, {}};
    s.p.batch = 3;
    s.p.Hq = 16;
    s.p.Hkv = 4;
    s.p.w = 16;
    for (int i = 0; i < 12; ++i) s.budgets.push_back((i * 97) % 700);
    shapes.push_back(s);
  }
  {
    Shape s{"one key", base_problem(), {}, {}};
    s.p.L = 1;
    s.p.w = 1;
    s.p.k = 1;
    shapes.push_back(s);
  }
  {
    Shape s{"wide pool 35 (unfused path)", base_problem(), {}, {}};
    s.p.pool = KVSEL_POOL_AVG;
    s.p.pool_kernel = 35;
    shapes.push_back(s);
  }
  {
    Shape s{"split row tile R=144", base_problem(), {}, {}};
    s.p.Hq = 16;
    s.p.Hkv = 2;
    s.p.w = 18;
    s.p.L = 1030;
    s.p.k = 60;
    shapes.push_back(s);
  }
  {
    Shape s{"DeferKV variant, mean query", base_problem(), {}, {}};
    s.p.has_decode = 1;
    s.p.weighting = 1;
    s.p.lambda = 0.1f;
    s.p.sink_tokens = 16;
    s.p.recent_tokens = 32;
    s.p.gqa = 1;
    shapes.push_back(s);
  }
  {
    Shape s{"streaming 8192", base_problem(), {}, {}};
    s.p.L = 32768;
    s.p.k = 2048;
    s.p.stream_keys = 8192;
    shapes.push_back(s);
  }
  {
    Shape s{"streaming 8192, pool 255 wide", base_problem(), {}, {}};
    s.p.L = 20000;
    s.p.k = 700;
    s.p.pool = 1;
    s.p.pool_kernel = 255;
    s.p.stream_keys = 8192;
    shapes.push_back(s);
  }
  {
    Shape s{"streaming 32768, row past the fused limit", base_problem(), {}, {}};
    s.p.L = 40000;
    s.p.k = 64;
    s.p.stream_keys = 32768;
    shapes.push_back(s);
  }
  {
    Shape s{"streaming 8192 over 2^20 keys", base_problem(), {}, {}};
    s.p.L = 1 << 20;
    s.p.k = 4096;
    s.p.key_chunk = 1024;
    s.p.stream_keys = 8192;
    shapes.push_back(s);
  }
  {
    Shape s{"2^20 keys", base_problem(), {}, {}};
    s.p.L = 1 << 20;
    s.p.k = 4096;
    shapes.push_back(s);
  }
  for (Shape &s : shapes) run_shape(s);

  // ---- the host-only greedy
  {
    const int32_t sizes[3] = {8, 16, 32};
    const double benefit[6] = {1.0, 1.5, 1.6, 0.5, 1.4, 2.0};
    int32_t out[2] = {-1, -1};
    check(kvsel_allocate_budgets(2, 3, sizes, benefit, 40, out) == KVSEL_OK, "allocate budgets");
    check(out[0] + out[1] <= 40 && out[0] >= 8 && out[1] >= 8, "allocate budgets: within the total");
    check(kvsel_allocate_budgets(2, 3, sizes, nullptr, 40, out) == KVSEL_EINVAL, "allocate budgets: NULL benefit");
  }

  const int stub_fail = reg_failures();
  std::printf("host ABI under sanitizers: %d checks failed, %d launch checks failed, %d launches checked\n", g_fail,
              stub_fail, reg_launches());
  return (g_fail == 0 && stub_fail == 0) ? 0 : 1;
}
