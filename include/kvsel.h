/*
 * kvsel -- attention-score-based KV-cache selection on AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library libkvsel.so.  All compute runs in hand-written HIP
 * kernels; every call validates its arguments on the host, then enqueues work
 * on the caller's stream and returns without synchronising.
 *
 * The operation, per sequence b and KV head h:
 *   1. observation rows: the last w prompt queries (positions L_b-w .. L_b-1),
 *      optionally followed by one decode-step query at position L_b
 *      (TideKV, "Delayed KV Eviction via Layer-Wise Chunked Prefill", §4.2,
 *      observation queries; DeferKV Guide, "Eviction Timing for KV Cache
 *      Compression", Phase 2, decode-aware observation window);
 *   2. logits s = scale * <q, k_i> for every prefix key i, causally masked for
 *      window rows (TideKV §4.2, Eq. (4) and the masking rule beside it);
 *   3. per-row softmax over the prefix, found with TideKV's two-pass blockwise
 *      procedure (§4.2): pass 1 streams key blocks keeping a running max and a
 *      rescaled sum of exponentials per row, pass 2 recomputes the logits;
 *   4. S[i] = sum over the G = Hq/Hkv query heads of group h and over the rows
 *      of c_r * p_r[i] (TideKV §4.2, grouped-query aggregation at KV-head
 *      granularity); c_r = 1 without a decode row, else 1-alpha for prompt
 *      rows and alpha for the decode row (DeferKV Guide, Phase 2 weighting),
 *      or the guide's exponential temporal weights (enum kvsel_weighting).
 *      With KVSEL_GQA_MEAN_QUERY the group's G heads are first averaged into
 *      one query per row (enum kvsel_gqa) and the sum over heads drops out;
 *   5. a stride-1 1-D pool of odd width (avg: zero-padded sum / width; max:
 *      over in-range positions) -- not defined on the pages;
 *   6. top-k: the min(k_bh, L_b) positions with the largest pooled score,
 *      lower position first among equal scores, reported ascending (TideKV
 *      §5 keeps original positions; DeferKV Guide, Phase 3, sorts them).
 *      Reserved positions (the first sink_tokens and the last recent_tokens
 *      of the sequence; DeferKV Guide, Phase 3) are kept before any other,
 *      lowest position first if the budget cannot hold them all, and the
 *      rest of the budget goes to the highest scores;
 *   7. gather of the kept K and V rows (TideKV §4.2 and §5, compact KV-head
 *      layout with per-head offsets, §4.1).
 * Query head g belongs to KV head g / G.
 *
 * Layouts (all packed, row-major, no padding):
 *   Q       bf16 [B][w'][Hq][d], w' = w + has_decode, decode row last.
 *   K, V    bf16 [sum_b L_b][Hkv][d]; sequence b occupies key rows
 *           seq_offsets[b] .. seq_offsets[b+1]-1 (token-major).
 *   scores, pooled
 *           fp32, segment (b,h) is L_b contiguous floats starting at
 *           Hkv*seq_offsets[b] + h*L_b.
 *   idx     int32 positions relative to the start of sequence b, ascending
 *           within each segment; segment (b,h) starts at out_offsets[b*Hkv+h]
 *           (from kvsel_plan) and holds min(k_bh, L_b) entries.
 *   K_out, V_out
 *           bf16 [sum of kept][d], same segments as idx (head-major within a
 *           sequence, i.e. the flattened variable-length layout).
 *
 * Ownership: the caller allocates and frees every buffer, including the
 * workspace (size from kvsel_plan).  The library never allocates, frees or
 * synchronises device memory.  Inputs are read-only.  The workspace needs no
 * initialisation and may be reused by later calls on the same stream; two
 * calls that overlap in time must not share a workspace.
 *
 * Errors: validation is synchronous and launches nothing when it fails.
 *   KVSEL_EINVAL       bad argument (see each function);
 *   KVSEL_EUNSUPPORTED valid but outside what this build implements
 *                      (d != 128, more than 64 KV heads, more than 512
 *                      observation rows per KV head, a sequence longer than
 *                      2^20 keys, device is not gfx950);
 *   KVSEL_EHIP         a HIP runtime call or kernel launch failed; the HIP
 *                      error text is available from kvsel_last_error().
 * No C++ exception crosses this interface.  NaN or Inf inputs give undefined
 * (but memory-safe) results.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVSEL_ABI_VERSION 2

/* Same type as hipStream_t; NULL means the default stream. */
typedef struct ihipStream_t *kvsel_stream_t;

typedef enum kvsel_status {
  KVSEL_OK = 0,
  KVSEL_EINVAL = 1,
  KVSEL_EUNSUPPORTED = 2,
  KVSEL_EHIP = 3
} kvsel_status;

typedef enum kvsel_pool {
  KVSEL_POOL_NONE = 0,
  KVSEL_POOL_AVG = 1,
  KVSEL_POOL_MAX = 2
} kvsel_pool;

/* Weights c_r of the observation rows in the aggregated score. */
typedef enum kvsel_weighting {
  /* 1 for every row without a decode row; with one, 1 - alpha for the prompt
   * rows and alpha for the decode row. */
  KVSEL_WEIGHT_ALPHA = 0,
  /* The DeferKV guide's exponential temporal weights (Phase 2): relative
   * positions r = -w+1 .. 0 for the prompt rows (oldest first) and r = 1 for
   * the decode row; c_r = exp(lambda * r) / sum over the rows of
   * exp(lambda * r'), so the weights sum to 1. */
  KVSEL_WEIGHT_EXP = 1
} kvsel_weighting;

/* How the Hq/Hkv query heads of a KV head's group enter the score. */
typedef enum kvsel_gqa {
  /* A softmax per query head, then the sum over the group's heads (TideKV
   * §4.2, scores aggregated at KV-head granularity). */
  KVSEL_GQA_SUM = 0,
  /* The DeferKV guide's shortcut (Phase 2 code): the group's queries are
   * averaged into one query per observation row, the mean rounded to the
   * nearest bf16 value (ties to even), and that row's softmax takes the
   * place of the G heads' sum.  A different score, at 1/G of the work. */
  KVSEL_GQA_MEAN_QUERY = 1
} kvsel_gqa;

/* Problem description, shared by every entry point.  Host memory. */
typedef struct kvsel_problem {
  int32_t batch;                 /* B >= 1 sequences */
  int32_t Hq;                    /* query heads, multiple of Hkv */
  int32_t Hkv;                   /* KV heads, 1..64 */
  int32_t d;                     /* head dim; this build: 128 */
  int64_t L;                     /* prefix length of every sequence when seq_offsets_h is NULL */
  const int64_t *seq_offsets_h;  /* host, B+1 increasing offsets into the key axis (first 0), or NULL */
  int32_t w;                     /* prompt observation rows, 1 <= w <= L_b for every b */
  int32_t has_decode;            /* 0 or 1: one extra decode-step row at position L_b */
  float alpha;                   /* decode weight in [0,1]; used only when has_decode */
  int32_t causal;                /* 1: window row at position p sees keys <= p; 0: all keys */
  float scale;                   /* logit scale; 0 selects 1/sqrt(d) */
  int32_t pool;                  /* kvsel_pool */
  int32_t pool_kernel;           /* odd, >= 1 (ignored for KVSEL_POOL_NONE) */
  int32_t k;                     /* uniform budget >= 0 when budgets_h is NULL */
  const int32_t *budgets_h;      /* host, B*Hkv budgets (>= 0, sequence-major), or NULL */
  int32_t key_chunk;             /* most keys per pass-1 statistics block (multiple of 32; TideKV's b_s);
                                    the library may use smaller blocks to fill the GPU (the result is
                                    the same up to the rounding order of the block merge); 0 = library choice */
  int32_t weighting;             /* a kvsel_weighting value; 0 is KVSEL_WEIGHT_ALPHA */
  float lambda;                  /* KVSEL_WEIGHT_EXP: finite, >= 0 (0 gives equal weights) */
  int32_t sink_tokens;           /* >= 0: positions 0 .. sink-1 of every sequence are always kept */
  int32_t recent_tokens;         /* >= 0: positions L_b-recent .. L_b-1 are always kept */
  int32_t gqa;                   /* a kvsel_gqa value; 0 is KVSEL_GQA_SUM */
  int32_t stream_keys;           /* 0, or a multiple of 2048: kvsel_compress's streaming form (below) */
} kvsel_problem;

/* KVSEL_ABI_VERSION of the loaded library. */
int kvsel_abi_version(void);

/*
 * Host-only planning.  Validates *p (pointer arguments are not needed) and
 * returns the workspace size, in bytes, that kvsel_score, kvsel_pool_topk
 * and kvsel_compress need for this problem (one size serves all three), and,
 * if out_offsets_h is not NULL, the B*Hkv+1 output segment offsets
 * (out_offsets_h[0] = 0, last = total kept rows): the compact layout of the
 * kept rows with per-head offsets (TideKV, "Delayed KV Eviction via
 * Layer-Wise Chunked Prefill", §4.1: each KV head keeps its own number of
 * tokens, stored flattened with offsets).  Segment (b, h) holds
 * min(k_bh, L_b) rows.
 * Errors: KVSEL_EINVAL for an invalid problem or NULL workspace_bytes.
 */
kvsel_status kvsel_plan(const kvsel_problem *p, size_t *workspace_bytes, int64_t *out_offsets_h);

/*
 * Steps 1-4: aggregated scores S (before pooling) into `scores`.
 * Q, K: device bf16 inputs; scores: device fp32 output; ws: device workspace
 * of at least kvsel_plan's size.  All device pointers 16-byte aligned.
 * Errors: KVSEL_EINVAL (invalid problem, NULL pointer, misalignment,
 * ws_bytes too small), KVSEL_EUNSUPPORTED, KVSEL_EHIP.
 */
kvsel_status kvsel_score(const kvsel_problem *p, const void *Q, const void *K, float *scores,
                         void *ws, size_t ws_bytes, kvsel_stream_t stream);

/*
 * The two passes of kvsel_score, for callers that schedule them separately
 * (and for measuring each).  kvsel_row_stats is TideKV's first pass (§4.2):
 * for every block of keys it records each observation row's running maximum
 * and rescaled sum of exponentials in the workspace.  kvsel_score_from_stats
 * merges those block records into each row's normaliser and runs the second
 * pass, which recomputes the logits and writes the aggregated scores S into
 * `scores`.  Calling kvsel_row_stats and then kvsel_score_from_stats on the
 * same stream, problem, inputs and workspace gives exactly the bytes of
 * kvsel_score; the workspace must not be used by any other call in between
 * (with KVSEL_GQA_MEAN_QUERY it also carries the mean queries, which
 * kvsel_row_stats forms and the second pass reads instead of Q).
 * Arguments and errors as for kvsel_score (kvsel_row_stats has no `scores`).
 */
kvsel_status kvsel_row_stats(const kvsel_problem *p, const void *Q, const void *K, void *ws, size_t ws_bytes,
                             kvsel_stream_t stream);
kvsel_status kvsel_score_from_stats(const kvsel_problem *p, const void *Q, const void *K, float *scores,
                                    void *ws, size_t ws_bytes, kvsel_stream_t stream);

/*
 * Steps 5-6: pool the given scores and select the top-k positions.
 * scores: device fp32 input (layout above); pooled: device fp32 output or
 * NULL (then it is kept in the workspace); idx: device int32 output.
 * Errors as for kvsel_score.
 */
kvsel_status kvsel_pool_topk(const kvsel_problem *p, const float *scores, float *pooled, int32_t *idx,
                             void *ws, size_t ws_bytes, kvsel_stream_t stream);

/*
 * Step 7: copy the rows named by idx (positions within each sequence) of K
 * and V into K_out and V_out.  An index outside [0, L_b) yields a zero row.
 * Needs no workspace.  Errors as for kvsel_score (no workspace checks).
 */
kvsel_status kvsel_gather(const kvsel_problem *p, const int32_t *idx, const void *K, const void *V,
                          void *K_out, void *V_out, kvsel_stream_t stream);

/*
 * Steps 1-7 in one call: idx, K_out, V_out and (if not NULL) pooled; the
 * unpooled scores stay in the workspace.
 *
 * With p->stream_keys = C > 0 (a multiple of 2048) it takes TideKV's
 * memory-bounded form instead (§4.2, two-pass blockwise streaming top-k):
 * the row statistics are gathered into a bounded number of states per
 * (sequence, KV head); pass 2 then visits the prefix C keys at a time
 * (plus the pool's half width on each side), pools the step's scores and
 * merges them into a running top-k of each (sequence, KV head).  With a
 * pool up to 33 wide and C plus the largest budget at most 16384, pass 1
 * runs once over the prefix with at most 64 states per (sequence, KV
 * head), a state folding ceil(L / 64) keys where that exceeds key_chunk;
 * otherwise pass 1 also visits the prefix C keys at a time, folding each
 * step's statistics into running ones.  The
 * workspace (kvsel_plan's size) then depends on C, the budgets, B, Hkv and
 * the rows, not on the prefix length; no whole-prefix score buffer exists,
 * so `pooled` must be NULL, and the other workspace entry points reject
 * such a problem (KVSEL_EINVAL).  C plus the largest budget must not exceed
 * 2^20.  The kept positions are those of the whole-prefix form, up to
 * positions whose pooled scores tie to within fp32 rounding (the row
 * statistics are merged in another order).
 */
kvsel_status kvsel_compress(const kvsel_problem *p, const void *Q, const void *K, const void *V,
                            int32_t *idx, void *K_out, void *V_out, float *pooled,
                            void *ws, size_t ws_bytes, kvsel_stream_t stream);

/*
 * kvsel_compress without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It allocates nothing: its
 * workspace is a 64 MiB array in device memory that the library holds on
 * each GPU it runs on, from the first call there until the process ends.
 * Arguments, layouts and results are those of kvsel_compress.
 *
 * Every call on one GPU uses that GPU's array, so calls that overlap on a
 * GPU (on other streams or host threads) race; order them.
 *
 * Errors as for kvsel_compress, and KVSEL_EUNSUPPORTED (message in
 * kvsel_last_error) for a problem whose kvsel_plan workspace exceeds
 * 64 MiB; KVSEL_EHIP if the array's device address cannot be obtained.
 */
kvsel_status kvsel_compress_noalloc(const kvsel_problem *p, const void *Q, const void *K, const void *V,
                                    int32_t *idx, void *K_out, void *V_out, float *pooled,
                                    kvsel_stream_t stream);

/*
 * Importance-guided warm-up (KVDrive, "A Holistic Multi-Tier KV Cache
 * Management System for Long-Context LLM Inference", §7.1): the observation
 * rows' attention over every prefix key, aggregated over the heads and the
 * layers of the model, ranks the prefix positions for placement in memory
 * tiers.
 *
 * kvsel_profile_layer: steps 1-4 for one layer's Q and K, then the sum of
 * S over the KV heads of each sequence, written to `profile` (accumulate =
 * 0) or added to it (accumulate = 1).  Calling it once per layer (the first
 * with 0) sums over the layers.  profile: device fp32 [sum_b L_b], sequence
 * b at seq_offsets[b], 16-byte aligned.  Every field of *p applies as for
 * kvsel_score; budgets, pool and reserved positions are not used.
 *
 * kvsel_tier_rank: pools the profile with the problem's pool kind and
 * width, ranks the positions of each sequence by descending pooled value
 * (the lower position first among equal values), and writes one label per
 * position to `tier` (device int8 [sum_b L_b], 16-byte aligned): 0 for the
 * first n_fast positions (GPU memory), 1 for the next n_mid (host memory),
 * 2 for the rest (the backing store only).  n_fast, n_mid >= 0; the tiers
 * simply run out on short sequences.  The problem's budgets, heads,
 * reserved positions and query fields are not used, but *p must be valid;
 * ws must hold kvsel_plan's size for *p.
 *
 * Errors as for kvsel_score; KVSEL_EINVAL also for accumulate not 0 or 1
 * and for a negative n_fast or n_mid.
 */
kvsel_status kvsel_profile_layer(const kvsel_problem *p, const void *Q, const void *K, float *profile,
                                 int32_t accumulate, void *ws, size_t ws_bytes, kvsel_stream_t stream);
kvsel_status kvsel_tier_rank(const kvsel_problem *p, const float *profile, int64_t n_fast, int64_t n_mid,
                             int8_t *tier, void *ws, size_t ws_bytes, kvsel_stream_t stream);

/*
 * Adaptive budgets from KVDrive's 2-D window scaling (§5.2): choose one size
 * per (layer, head) pair out of a few candidates to maximise the summed
 * benefit under a total budget.  Here a pair's size is its KV budget k and
 * its benefit the importance it keeps.
 *
 * kvsel_topk_mass: for each of the n_sizes candidate budgets sizes_h[j]
 * (host, >= 0), the sum of the min(sizes_h[j], L_b) largest values of every
 * (sequence, KV head) segment of `pooled` (device fp32, the layout of
 * kvsel_pool_topk's pooled output), into mass (device fp32
 * [B*Hkv][n_sizes], segment-major).  The kept set is exactly the top-k of
 * the given fp32 values (ties to the lower position); the sum is fp32 in a
 * fixed order.  The problem's pool, budgets and reserved positions are not
 * used; ws must hold kvsel_plan's size for *p.
 *
 * kvsel_allocate_budgets (host only, no device): the greedy of §5.2.  Every
 * one of the n_items pairs starts at sizes_h[0] (strictly increasing,
 * >= 0); while some pair's next size fits what is left of `total` and adds
 * benefit, the step with the largest (added benefit) / (added entries) is
 * taken, the lower pair index first on equal ratios.  benefit_h: host
 * double [n_items][n_sizes], finite.  budgets_h (host int32 [n_items]):
 * the chosen size of every pair (sizes_h[0] everywhere if even those exceed
 * total), ready to be a layer's budgets_h.
 *
 * Errors: KVSEL_EINVAL for NULL or invalid arguments (and as for
 * kvsel_pool_topk in kvsel_topk_mass).
 */
kvsel_status kvsel_topk_mass(const kvsel_problem *p, const float *pooled, int32_t n_sizes, const int32_t *sizes_h,
                             float *mass, void *ws, size_t ws_bytes, kvsel_stream_t stream);
kvsel_status kvsel_allocate_budgets(int32_t n_items, int32_t n_sizes, const int32_t *sizes_h,
                                    const double *benefit_h, int64_t total, int32_t *budgets_h);

/* Static text for a status code. */
const char *kvsel_status_string(kvsel_status s);

/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char *kvsel_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
