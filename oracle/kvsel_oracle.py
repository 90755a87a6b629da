"""Plain fp64 CPU oracle for attention-score-based KV-cache selection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library; it is written from the definitions on the pages,
slowly and obviously, in float64 numpy.

What it computes (one sequence ``b`` and one KV head ``h`` at a time):

1. Observation rows.  The last ``w`` prompt positions ``L-w .. L-1`` form the
   window; optionally one decode-step row sits at position ``L`` and sees every
   prefix key.  (SnapKV-style observation window: TideKV, "Delayed KV Eviction
   via Layer-Wise Chunked Prefill", §4.2; decode-aware window: "DeferKV Guide:
   Eviction Timing for KV Cache Compression", section "Phase 2: The
   Decode-Aware Observation Window and Temporal Weighting".)
2. Logits ``s[r, i] = scale * <q_r, k_i>`` with ``scale = 1/sqrt(d)`` by
   default (TideKV §4.2, Eq. (4) -- the formula itself is missing from the
   extracted page; the DeferKV guide's code divides by sqrt(d)).
3. Causal visibility: a window row at position ``p`` sees keys ``i <= p``
   (TideKV §4.2: keys beyond a query's causal position get -inf).  The decode
   row sees all ``L`` prefix keys.
4. Per-row softmax over the visible keys, computed with an explicit max and
   sum (the plain definition; TideKV's blockwise two-pass procedure reaches the
   same values, §4.2, and ``blockwise_row_stats`` below restates it).
5. Aggregation: ``S[i] = sum_{g in group h} sum_r c_r * P_{g,r}[i]`` -- per
   query-head softmax, then a sum over the group's query heads (TideKV §4.2:
   scores aggregated at KV-head granularity) and over the window rows.  Row
   weights ``c_r = 1`` without a decode row; with one, ``1 - alpha`` for the
   prompt rows and ``alpha`` for the decode row (the DeferKV guide's
   prompt-vs-decode weighting, in its two-level form).  Optionally the
   guide's exponential temporal weights instead: ``c_r`` proportional to
   ``exp(lambda * r)`` over relative row positions ``r = -w+1 .. 0`` (and ``1``
   for the decode row), normalised to sum to 1.  Optionally the guide's
   grouped-query shortcut instead of the per-head sum: the group's queries
   are averaged into one query per row first (the mean rounded once to
   bfloat16, the dtype of the queries it averages), and that single row's
   softmax is weighted and summed over the rows.
6. 1-D pool of odd width ``K`` and stride 1 (no page defines it; reading:
   ``avg`` = zero-padded window sum divided by ``K``, ``max`` = max over the
   in-range positions only).
7. Top-k: order positions by (descending score, ascending index) and keep the
   first ``min(k, L)``; return them in ascending position order (the DeferKV
   guide sorts the kept indices; TideKV keeps original positions, §5).
   Optionally the guide's reserved positions (Phase 3): the first ``sink`` and
   the last ``recent`` positions are kept before any other, lowest position
   first, and the rest of the budget goes to the highest scores.
8. Gather: the kept rows of K and V, copied exactly (TideKV §4.2 and §5).

Also the warm-up placement of "KVDrive: A Holistic Multi-Tier KV Cache
Management System for Long-Context LLM Inference" (§7.1, importance-guided
warm-up): the aggregated scores of step 5, summed over the KV heads of a
sequence and over the model's layers, give one importance value per prefix
position (``importance_profile``); ranked by (descending importance,
ascending position), the first ``n_fast`` positions go to the fastest tier
(GPU memory), the next ``n_mid`` to the middle tier (host memory) and the
rest stay in the backing store only (``tier_labels``).

TideKV's memory-bounded form of steps 4-7 (§4.2) is ``streaming_select``:
pass 1 as in ``blockwise_row_stats``; pass 2 visits the key blocks in order,
scores (and pools) one block at a time and merges its positions into a
running top-k, so no per-position buffer over the whole prefix is kept.  It
reaches the same selection as ``select_topk`` on the whole pooled score.

And adaptive budgets: KVDrive's 2-D window scaling (§5.2) chooses one size
per (layer, head) from a few candidates to maximise the summed benefit under
a total memory budget, with a greedy rule that starts every pair at its
smallest size and repeatedly enlarges the pair whose next step has the
highest benefit-to-cost ratio (``greedy_allocate``).  Here a pair's size is
its KV budget ``k`` (cost ``k`` entries) and its benefit the importance it
keeps, the sum of its ``k`` largest pooled scores (``topk_mass``).

Query-head ``g`` belongs to KV head ``g // G`` with ``G = Hq // Hkv``
(consecutive grouping, as the DeferKV guide's code reshapes the heads).

Every function is pinned by tests that do not call it to check itself:
hand-worked 8-token examples with closed-form values, closed forms for
constant queries, the row-sum invariant, brute-force full causal attention,
library pooling routines, exhaustive subset enumeration for top-k and
``numpy.take`` for the gather.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "observation_positions",
    "visible_mask",
    "row_weights",
    "temporal_row_weights",
    "protected_mask",
    "row_probabilities",
    "round_to_bf16",
    "mean_query_rows",
    "head_scores",
    "pool1d",
    "select_topk",
    "gather_rows",
    "blockwise_row_stats",
    "blockwise_head_scores",
    "plan_offsets",
    "compress",
    "importance_profile",
    "tier_labels",
    "topk_mass",
    "greedy_allocate",
    "streaming_select",
]


def _check_finite(*arrays):
    for a in arrays:
        if not np.all(np.isfinite(a)):
            raise ValueError("oracle inputs must be finite (NaN/Inf are undefined)")


def observation_positions(L: int, w: int, has_decode: bool) -> np.ndarray:
    """Absolute positions of the observation rows of one sequence.

    Window rows are the last ``w`` prompt positions ``L-w .. L-1``; the
    optional decode-step row follows at position ``L`` (DeferKV guide, Phase 2;
    TideKV §4.2 observation queries).
    """
    if not (1 <= w <= L):
        raise ValueError("need 1 <= w <= L")
    pos = list(range(L - w, L))
    if has_decode:
        pos.append(L)
    return np.asarray(pos, dtype=np.int64)


def visible_mask(positions: np.ndarray, L: int, causal: bool) -> np.ndarray:
    """Boolean [rows, L]: which prefix keys each observation row may attend to.

    With ``causal`` a row at position ``p`` sees keys ``i <= p`` (TideKV §4.2);
    a decode row (``p == L``) therefore sees all ``L`` keys.  Without
    ``causal`` every row sees every prefix key (the DeferKV guide's code).
    """
    keys = np.arange(L)[None, :]
    if causal:
        return keys <= positions[:, None]
    return np.ones((len(positions), L), dtype=bool)


def row_weights(w: int, has_decode: bool, alpha: float) -> np.ndarray:
    """Weights ``c_r`` of the observation rows.

    All ones for a prompt-only window; with a decode row, ``1 - alpha`` for
    each prompt row and ``alpha`` for the decode row.
    """
    if not has_decode:
        return np.ones(w, dtype=np.float64)
    c = np.full(w + 1, 1.0 - alpha, dtype=np.float64)
    c[w] = alpha
    return c


def temporal_row_weights(w: int, has_decode: bool, lam: float) -> np.ndarray:
    """Exponential temporal weights of the observation rows (DeferKV guide,
    Phase 2, temporal weighting).

    Row ``j`` of the prompt window (position ``L - w + j``) has relative
    position ``r = j - (w - 1)``, from ``-w + 1`` up to ``0``; the decode row has
    ``r = 1``.  ``c_r = exp(lam * r) / sum over the rows of exp(lam * r')``, so
    the weights sum to 1 and the latest row weighs most.
    """
    r = np.arange(w, dtype=np.float64) - (w - 1)
    if has_decode:
        r = np.append(r, 1.0)
    e = np.exp(lam * (r - r.max()))
    return e / e.sum()


def protected_mask(L: int, sink: int, recent: int) -> np.ndarray:
    """Positions kept whatever their score (DeferKV guide, Phase 3): the first
    ``sink`` prefix positions (attention sinks) and the last ``recent`` ones
    (the recent window)."""
    keep = np.zeros(L, dtype=bool)
    keep[:max(0, min(int(sink), L))] = True
    if recent > 0:
        keep[max(0, L - int(recent)):] = True
    return keep


def row_probabilities(q_rows: np.ndarray, K_h: np.ndarray, vis: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention probabilities of each observation row over the prefix.

    ``q_rows`` [R, d], ``K_h`` [L, d], ``vis`` [R, L] -> P [R, L] with
    ``P[r, i] = exp(s[r,i] - M_r) / sum_{j visible} exp(s[r,j] - M_r)`` on the
    visible keys and 0 elsewhere, ``s = scale * q_rows @ K_h.T``.
    """
    logits = scale * (q_rows @ K_h.T)
    masked = np.where(vis, logits, -np.inf)
    m = masked.max(axis=1, keepdims=True)
    e = np.where(vis, np.exp(masked - m), 0.0)
    z = e.sum(axis=1, keepdims=True)
    return e / z


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range, so its
    spacing at ``|x|`` in ``[2^e, 2^(e+1))`` is ``2^(e-7)`` (never below the
    subnormal spacing ``2^-133``).  Each value is divided by its spacing,
    rounded to an integer with ties to even (``numpy.rint``) and scaled back.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    _, e = np.frexp(x[nz])  # |x| = m * 2^e with 0.5 <= m < 1, so |x| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)  # exponent of the spacing
    out[nz] = np.ldexp(np.rint(np.ldexp(x[nz], -q)), q)
    return out


def mean_query_rows(Q_b: np.ndarray, h: int, G: int) -> np.ndarray:
    """The DeferKV guide's grouped-query shortcut (Phase 2 code): one query
    per observation row, the mean of the ``G`` query heads of group ``h``,
    rounded to bfloat16 like the queries it averages.  [w', Hq, d] -> [w', d]."""
    return round_to_bf16(Q_b[:, h * G:(h + 1) * G, :].mean(axis=1))


def head_scores(Q_b: np.ndarray, K_b: np.ndarray, h: int, Hkv: int, *, w: int, has_decode: bool,
                alpha: float, causal: bool, scale: float, weighting: str = "alpha", lam: float = 0.0,
                gqa: str = "sum") -> np.ndarray:
    """Aggregated importance ``S[i]`` of one (sequence, KV head).

    ``Q_b`` [w', Hq, d] observation queries of the sequence (decode row last),
    ``K_b`` [L, Hkv, d] its keys.  Sums ``c_r * P`` over the window rows and the
    ``G`` query heads of group ``h`` (``gqa`` "sum"), or over the rows of the
    group's mean query (``gqa`` "mean", see ``mean_query_rows``); ``c_r`` from
    ``row_weights`` (weighting "alpha") or ``temporal_row_weights`` (weighting
    "exp").
    """
    L = K_b.shape[0]
    Hq = Q_b.shape[1]
    G = Hq // Hkv
    pos = observation_positions(L, w, has_decode)
    vis = visible_mask(pos, L, causal)
    if weighting == "alpha":
        c = row_weights(w, has_decode, alpha)
    elif weighting == "exp":
        c = temporal_row_weights(w, has_decode, lam)
    else:
        raise ValueError(f"unknown weighting {weighting!r}")
    K_h = K_b[:, h, :]
    if gqa == "sum":
        query_sets = [Q_b[:, h * G + gi, :] for gi in range(G)]
    elif gqa == "mean":
        query_sets = [mean_query_rows(Q_b, h, G)]
    else:
        raise ValueError(f"unknown gqa {gqa!r}")
    S = np.zeros(L, dtype=np.float64)
    for q in query_sets:
        P = row_probabilities(q, K_h, vis, scale)
        S += (c[:, None] * P).sum(axis=0)
    return S


def pool1d(S: np.ndarray, kind: str, kernel: int) -> np.ndarray:
    """Stride-1, odd-width 1-D pool producing one value per position.

    ``avg``: sum of ``S[j]`` for ``j`` in ``[i-r, i+r]`` (positions outside the
    sequence count as 0) divided by ``kernel``; ``max``: maximum over the
    positions of that window that lie inside the sequence; ``none``: identity.
    ``r = (kernel - 1) // 2``.
    """
    if kernel < 1 or kernel % 2 == 0:
        raise ValueError("pool kernel must be odd and >= 1")
    L = S.shape[0]
    if kind == "none" or kernel == 1:
        return S.copy()
    r = (kernel - 1) // 2
    out = np.empty(L, dtype=np.float64)
    for i in range(L):
        lo, hi = max(0, i - r), min(L, i + r + 1)
        if kind == "avg":
            out[i] = S[lo:hi].sum() / kernel
        elif kind == "max":
            out[i] = S[lo:hi].max()
        else:
            raise ValueError(f"unknown pool kind {kind!r}")
    return out


def select_topk(P: np.ndarray, k: int, protected=None) -> np.ndarray:
    """Positions of the ``min(k, L)`` largest values, ascending.

    Ordering is by descending value, then ascending position, so among equal
    values the lower position is kept.  Positions flagged in ``protected``
    (a boolean mask) come before every other position, in ascending order
    among themselves, so they are kept first and the rest of the budget goes
    to the highest-scoring others (the DeferKV guide's reserved sinks and
    recent window, Phase 3).
    """
    L = P.shape[0]
    keff = max(0, min(int(k), L))
    prot = np.zeros(L, dtype=bool) if protected is None else np.asarray(protected, dtype=bool)
    # lexsort: the last key is primary -- protected first, then -P (only for
    # the unprotected), then position
    order = np.lexsort((np.arange(L), np.where(prot, 0.0, -P), ~prot))
    return np.sort(order[:keff]).astype(np.int64)


def gather_rows(X_b: np.ndarray, idx: np.ndarray, h: int) -> np.ndarray:
    """Rows ``X_b[idx, h, :]`` (exact copies) of one sequence and KV head."""
    return X_b[idx, h, :].copy()


def blockwise_row_stats(q_rows: np.ndarray, K_h: np.ndarray, vis: np.ndarray, scale: float,
                        block: int):
    """TideKV pass 1 (§4.2): streaming max / sum of exponentials per row.

    Keys are visited in blocks of ``block``; for every row the running maximum
    ``m`` and the running sum ``Z`` of ``exp(s - m)`` are updated block by
    block, rescaling the previous sum whenever the maximum grows (the online
    normaliser of Milakov & Gimelshein, 2018).  Returns ``(M, Z)`` per row.
    """
    R, L = vis.shape
    m = np.full(R, -np.inf)
    Z = np.zeros(R)
    for start in range(0, L, block):
        stop = min(L, start + block)
        s = scale * (q_rows @ K_h[start:stop].T)
        v = vis[:, start:stop]
        s = np.where(v, s, -np.inf)
        bm = s.max(axis=1)
        new_m = np.maximum(m, bm)
        for r in range(R):
            if new_m[r] == -np.inf:
                continue  # nothing visible yet for this row
            rescale = np.exp(m[r] - new_m[r]) if m[r] != -np.inf else 0.0
            Z[r] = Z[r] * rescale + np.exp(s[r][v[r]] - new_m[r]).sum()
            m[r] = new_m[r]
    return m, Z


def blockwise_head_scores(Q_b: np.ndarray, K_b: np.ndarray, h: int, Hkv: int, *, w: int,
                          has_decode: bool, alpha: float, causal: bool, scale: float,
                          block: int) -> np.ndarray:
    """TideKV's two-pass blockwise scoring (§4.2) for one (sequence, KV head).

    Pass 1 gathers ``(M_r, Z_r)`` with :func:`blockwise_row_stats`; pass 2
    revisits the key blocks, recomputes the logits and adds
    ``c_r * exp(s - M_r) / Z_r`` into the per-key sum.  Mathematically equal
    to :func:`head_scores`.
    """
    L = K_b.shape[0]
    Hq = Q_b.shape[1]
    G = Hq // Hkv
    pos = observation_positions(L, w, has_decode)
    vis = visible_mask(pos, L, causal)
    c = row_weights(w, has_decode, alpha)
    K_h = K_b[:, h, :]
    S = np.zeros(L)
    for gi in range(G):
        q = Q_b[:, h * G + gi, :]
        M, Z = blockwise_row_stats(q, K_h, vis, scale, block)
        for start in range(0, L, block):
            stop = min(L, start + block)
            s = scale * (q @ K_h[start:stop].T)
            p = np.where(vis[:, start:stop], np.exp(s - M[:, None]), 0.0) / Z[:, None]
            S[start:stop] += (c[:, None] * p).sum(axis=0)
    return S


def plan_offsets(seq_lens, Hkv: int, budgets) -> np.ndarray:
    """Output segment offsets: segment ``(b, h)`` holds ``min(k_bh, L_b)`` rows.

    Segments are ordered sequence-major, head-minor; returns ``B*Hkv + 1``
    prefix offsets (TideKV §4.1: head-adaptive budgets give a flattened
    variable-length layout with per-head offsets).
    """
    out = [0]
    for b, L in enumerate(seq_lens):
        for h in range(Hkv):
            out.append(out[-1] + max(0, min(int(budgets[b][h]), int(L))))
    return np.asarray(out, dtype=np.int64)


def compress(Q, K, V, *, seq_lens, Hq: int, Hkv: int, w: int, has_decode: bool = False,
             alpha: float = 0.0, causal: bool = True, scale=None, pool: str = "none",
             pool_kernel: int = 1, k=None, budgets=None, heads=None, weighting: str = "alpha",
             lam: float = 0.0, sink: int = 0, recent: int = 0, gqa: str = "sum"):
    """Whole path for a packed batch.

    ``Q`` [B, w', Hq, d]; ``K``, ``V`` [sum L_b, Hkv, d] (sequences packed
    back to back); float64 arrays holding the exact bf16 input values.  Either a
    uniform ``k`` or ``budgets`` [B][Hkv].  ``heads`` optionally restricts the
    work to a list of ``(b, h)`` pairs (the others are left out of the result).

    Returns a dict keyed by ``(b, h)`` with ``scores``, ``pooled``, ``idx``,
    ``K_out`` and ``V_out``, plus ``out_offsets``.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    _check_finite(Q, K, V)
    B = len(seq_lens)
    d = K.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if budgets is None:
        budgets = [[k] * Hkv for _ in range(B)]
    starts = np.concatenate([[0], np.cumsum(seq_lens)])
    want = set(heads) if heads is not None else None
    res = {"out_offsets": plan_offsets(seq_lens, Hkv, budgets)}
    for b in range(B):
        K_b = K[starts[b]:starts[b + 1]]
        V_b = V[starts[b]:starts[b + 1]]
        for h in range(Hkv):
            if want is not None and (b, h) not in want:
                continue
            S = head_scores(Q[b], K_b, h, Hkv, w=w, has_decode=has_decode, alpha=alpha,
                            causal=causal, scale=scale, weighting=weighting, lam=lam, gqa=gqa)
            P = pool1d(S, pool, pool_kernel)
            idx = select_topk(P, budgets[b][h], protected_mask(len(S), sink, recent))
            res[(b, h)] = {
                "scores": S,
                "pooled": P,
                "idx": idx,
                "K_out": gather_rows(K_b, idx, h),
                "V_out": gather_rows(V_b, idx, h),
            }
    return res


def importance_profile(layers, *, seq_lens, Hq: int, Hkv: int, w: int, has_decode: bool = False,
                       alpha: float = 0.0, causal: bool = True, scale=None, weighting: str = "alpha",
                       lam: float = 0.0, gqa: str = "sum"):
    """KVDrive §7.1: the importance of every prefix position, the observation
    rows' attention aggregated over all heads and all layers.

    ``layers``: a list of ``(Q, K)`` pairs, one per layer, in the layouts of
    :func:`compress` (float64 arrays holding the bf16 input values).  Each
    layer contributes the aggregated score ``S`` of every KV head
    (:func:`head_scores`); returns one float64 array of length ``L_b`` per
    sequence with the sum over layers and KV heads.
    """
    B = len(seq_lens)
    starts = np.concatenate([[0], np.cumsum(seq_lens)])
    prof = [np.zeros(int(L)) for L in seq_lens]
    for Q, K in layers:
        Q = np.asarray(Q, dtype=np.float64)
        K = np.asarray(K, dtype=np.float64)
        _check_finite(Q, K)
        sc = (1.0 / np.sqrt(K.shape[2])) if scale is None else scale
        for b in range(B):
            K_b = K[starts[b]:starts[b + 1]]
            for h in range(Hkv):
                prof[b] += head_scores(Q[b], K_b, h, Hkv, w=w, has_decode=has_decode, alpha=alpha,
                                       causal=causal, scale=sc, weighting=weighting, lam=lam, gqa=gqa)
    return prof


def tier_labels(profile: np.ndarray, n_fast: int, n_mid: int, pool: str = "none", pool_kernel: int = 1):
    """KVDrive §7.1 placement of one sequence: rank the (optionally pooled)
    importance values, highest first and the lower position first among
    equal values; rank < n_fast -> tier 0 (GPU memory), rank < n_fast + n_mid
    -> tier 1 (host memory), otherwise tier 2 (the backing store only).
    Returns int8 labels, one per position."""
    P = pool1d(np.asarray(profile, dtype=np.float64), pool, pool_kernel)
    L = len(P)
    order = np.lexsort((np.arange(L), -P))  # last key first: descending value, then ascending position
    rank = np.empty(L, dtype=np.int64)
    rank[order] = np.arange(L)
    labels = np.full(L, 2, dtype=np.int8)
    labels[rank < int(n_fast) + int(n_mid)] = 1
    labels[rank < int(n_fast)] = 0
    return labels


def topk_mass(P: np.ndarray, sizes) -> np.ndarray:
    """Importance kept by a budget: for each candidate ``k`` in ``sizes``, the
    sum of the ``min(k, L)`` largest values of ``P``."""
    desc = np.sort(np.asarray(P, dtype=np.float64))[::-1]
    cum = np.concatenate([[0.0], np.cumsum(desc)])
    return np.array([cum[min(int(k), len(desc))] for k in sizes])


def greedy_allocate(benefit, sizes, total: int) -> np.ndarray:
    """KVDrive §5.2's greedy for the multiple-choice knapsack.

    ``benefit`` [items][len(sizes)]: benefit of each candidate size (sizes
    ascending, the cost of a size is the size itself); ``total``: the budget.
    Every item starts at its smallest size.  While some item's next size
    fits the remaining budget and adds benefit, the one with the largest
    (added benefit) / (added cost) is enlarged by one step; equal ratios go to
    the lower item index.  Returns the chosen size index of every item
    (all 0 if even the smallest sizes exceed the budget).
    """
    benefit = np.asarray(benefit, dtype=np.float64)
    sizes = [int(x) for x in sizes]
    n = benefit.shape[0]
    choice = np.zeros(n, dtype=np.int64)
    left = int(total) - n * sizes[0]
    if left < 0:
        return choice
    while True:
        best, best_ratio = -1, 0.0
        for i in range(n):
            j = choice[i]
            if j + 1 >= len(sizes):
                continue
            dc = sizes[j + 1] - sizes[j]
            db = benefit[i, j + 1] - benefit[i, j]
            if dc > left or db <= 0.0:
                continue
            ratio = db / dc if dc > 0 else np.inf
            if ratio > best_ratio:
                best, best_ratio = i, ratio
        if best < 0:
            return choice
        left -= sizes[choice[best] + 1] - sizes[choice[best]]
        choice[best] += 1


def streaming_select(Q_b: np.ndarray, K_b: np.ndarray, h: int, Hkv: int, *, w: int, has_decode: bool,
                     alpha: float, causal: bool, scale: float, block: int, k: int, pool: str = "none",
                     pool_kernel: int = 1, weighting: str = "alpha", lam: float = 0.0, gqa: str = "sum",
                     sink: int = 0, recent: int = 0) -> np.ndarray:
    """TideKV §4.2's two-pass blockwise streaming top-k for one (sequence, KV head).

    Pass 1 collects each observation row's (M, Z) over the key blocks.  Pass 2
    walks the blocks in order; for block [s, e) it recomputes the normalised
    probabilities of the keys [s - r, e + r) (r = the pool's half width, so
    the pool of every position of the block sees its real neighbours), forms
    the block's aggregated and pooled scores, and keeps the best ``k`` of
    (running top-k) + (block positions), ordered as ``select_topk`` orders
    them.  The memory held besides one block is the running top-k.  Returns
    the kept positions ascending.
    """
    L = K_b.shape[0]
    Hq = Q_b.shape[1]
    G = Hq // Hkv
    pos = observation_positions(L, w, has_decode)
    vis = visible_mask(pos, L, causal)
    c = row_weights(w, has_decode, alpha) if weighting == "alpha" else temporal_row_weights(w, has_decode, lam)
    K_h = K_b[:, h, :]
    if gqa == "sum":
        query_sets = [Q_b[:, h * G + gi, :] for gi in range(G)]
    else:
        query_sets = [mean_query_rows(Q_b, h, G)]
    stats = [blockwise_row_stats(q, K_h, vis, scale, block) for q in query_sets]
    r = 0 if pool == "none" else (pool_kernel - 1) // 2
    prot_all = protected_mask(L, sink, recent)
    keep = max(0, min(int(k), L))
    run_val = np.zeros(0)
    run_pos = np.zeros(0, dtype=np.int64)
    for start in range(0, L, block):
        stop = min(L, start + block)
        lo, hi = max(0, start - r), min(L, stop + r)
        S = np.zeros(hi - lo)
        for q, (M, Z) in zip(query_sets, stats):
            logits = scale * (q @ K_h[lo:hi].T)
            pr = np.where(vis[:, lo:hi], np.exp(logits - M[:, None]), 0.0) / Z[:, None]
            S += (c[:, None] * pr).sum(axis=0)
        # pool the block's positions from S on [lo, hi); outside [0, L) as in pool1d
        P = np.empty(stop - start)
        for i in range(start, stop):
            a, b = i - r, i + r + 1
            win = S[max(a, lo) - lo:min(b, hi) - lo]
            if pool == "avg":
                P[i - start] = win.sum() / pool_kernel
            elif pool == "max":
                P[i - start] = win.max()
            else:
                P[i - start] = S[i - lo]
        val = np.concatenate([run_val, P])
        cand = np.concatenate([run_pos, np.arange(start, stop)])
        prot = prot_all[cand]
        order = np.lexsort((cand, np.where(prot, 0.0, -val), ~prot))[:keep]
        run_val, run_pos = val[order], cand[order]
    return np.sort(run_pos)
