"""Pins of the fp64 oracle against facts that do not come from the oracle.

Closed forms are evaluated here with ``math``; brute force uses scipy's and
torch's own attention/softmax routines; top-k uses exhaustive enumeration;
pooling uses torch's pooling routines.  The ``mutation`` tests plant plausible
mistakes in the oracle (on the CPU) and check that some pin catches each one.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle.kvsel_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
E = math.e


def _hand():
    with open(GOLDEN) as f:
        return json.load(f)


def _closed_forms():
    """Expected aggregated scores S of the hand examples (before pooling)."""
    Z = 2 * E**2 + E + 5  # row at position 7, q=+1: logits [2,0,0,1,0,0,0,2]
    a, b, c = E**2 / Z, 1 / Z, E / Z
    p_plus = [a, b, b, c, b, b, b, a]
    Z6 = E**2 + E + 5  # row at position 6 sees keys 0..6 only
    p6 = [E**2 / Z6, 1 / Z6, 1 / Z6, E / Z6, 1 / Z6, 1 / Z6, 1 / Z6, 0.0]
    Zm = 2 * math.exp(-2) + math.exp(-1) + 5  # q=-1: logits [-2,0,0,-1,0,0,0,-2]
    p_minus = [math.exp(-2) / Zm, 1 / Zm, 1 / Zm, math.exp(-1) / Zm, 1 / Zm, 1 / Zm, 1 / Zm, math.exp(-2) / Zm]
    return {
        "ex1": p_plus,
        "ex2": [x + y for x, y in zip(p6, p_plus)],
        "ex3": [x + y for x, y in zip(p_plus, p_minus)],
        "ex4": [0.5 * x + 0.5 * y for x, y in zip(p_plus, p_minus)],
        "ex4_a025": [0.75 * x + 0.25 * y for x, y in zip(p_plus, p_minus)],
        "p_plus": p_plus,
        "p_minus": p_minus,
    }


def _run_hand(ex, keys_c0, d=128, alpha=None, scale=1.0):
    L = len(keys_c0)
    Hq, Hkv = ex["Hq"], ex["Hkv"]
    K = np.zeros((L, Hkv, d))
    K[:, :, 0] = np.asarray(keys_c0, dtype=float)[:, None]
    V = np.zeros((L, Hkv, d))
    V[:, :, 0] = np.arange(L)[:, None]
    Q = np.zeros((1, len(ex["q_c0"]), Hq, d))
    Q[0, :, :, 0] = np.asarray(ex["q_c0"], dtype=float)
    return O.compress(Q, K, V, seq_lens=[L], Hq=Hq, Hkv=Hkv, w=ex["w"], has_decode=ex["has_decode"],
                      alpha=ex["alpha"] if alpha is None else alpha, causal=ex["causal"], scale=scale,
                      pool=ex["pool"], pool_kernel=ex["pool_kernel"], k=ex["k"])


def _expected_scores(name):
    cf = _closed_forms()
    if name.startswith("ex1"):
        return cf["ex1"]
    return cf[name[:3]]


def _expected_pooled(ex):
    S = _expected_scores(ex["name"])
    L, K = len(S), ex["pool_kernel"]
    r = (K - 1) // 2
    if ex["pool"] == "none":
        return S
    out = []
    for i in range(L):
        win = [S[j] for j in range(i - r, i + r + 1) if 0 <= j < L]
        out.append(sum(win) / K if ex["pool"] == "avg" else max(win))
    return out


# ---------------------------------------------------------------- hand examples
@pytest.mark.parametrize("ex", _hand()["examples"], ids=lambda e: e["name"])
def test_hand_examples(ex):
    keys = _hand()["keys_c0"]
    res = _run_hand(ex, keys)[(0, 0)]
    np.testing.assert_allclose(res["scores"], _expected_scores(ex["name"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(res["pooled"], _expected_pooled(ex), rtol=0, atol=1e-13)
    assert res["idx"].tolist() == ex["expect_idx"]


def test_hand_values_printed_in_blueprint():
    """Six-digit values of the hand examples, as derived by hand."""
    cf = _closed_forms()
    np.testing.assert_allclose(cf["ex1"][:4], [0.328455, 0.044452, 0.044452, 0.120832], atol=1e-6)
    np.testing.assert_allclose(cf["ex2"][:4], [0.817559, 0.110645, 0.110645, 0.300763], atol=1e-6)
    np.testing.assert_allclose(cf["ex3"][:4], [0.352457, 0.221802, 0.221802, 0.186076], atol=1e-6)
    np.testing.assert_allclose(sum(cf["ex3"]), 2.0, atol=1e-14)
    np.testing.assert_allclose(sum(cf["ex4"]), 1.0, atol=1e-14)


def test_decode_weight_asymmetric():
    ex = [e for e in _hand()["examples"] if e["name"].startswith("ex4")][0]
    res = _run_hand(ex, _hand()["keys_c0"], alpha=0.25)[(0, 0)]
    np.testing.assert_allclose(res["scores"], _closed_forms()["ex4_a025"], atol=1e-13)


def test_default_scale_is_inverse_sqrt_d():
    # d = 64: scale 1/8, so q = 8 reproduces the unit-scale logits of example 1.
    ex = dict(_hand()["examples"][0])
    ex["q_c0"] = [[8]]
    res = _run_hand(ex, _hand()["keys_c0"], d=64, scale=None)[(0, 0)]
    np.testing.assert_allclose(res["scores"], _closed_forms()["ex1"], atol=1e-13)


def test_consecutive_query_head_grouping():
    # KV head 0 holds the example keys, KV head 1 all-zero keys.  Query heads
    # 0,1 (group 0) use q=+1; heads 2,3 (group 1) use q=-1.
    L, d = 8, 128
    K = np.zeros((L, 2, d))
    K[:, 0, 0] = _hand()["keys_c0"]
    Q = np.zeros((1, 1, 4, d))
    Q[0, 0, :2, 0] = 1.0
    Q[0, 0, 2:, 0] = -1.0
    res = O.compress(Q, K, K, seq_lens=[L], Hq=4, Hkv=2, w=1, scale=1.0, k=8)
    np.testing.assert_allclose(res[(0, 0)]["scores"], [2 * x for x in _closed_forms()["p_plus"]], atol=1e-13)
    np.testing.assert_allclose(res[(0, 1)]["scores"], [2 / 8] * 8, atol=1e-14)


# ---------------------------------------------------------------- closed forms and invariants
def test_zero_queries_give_uniform_rows():
    L, d = 8, 16
    rng = np.random.default_rng(0)
    K = rng.standard_normal((L, 1, d))
    Q = np.zeros((1, 2, 1, d))
    res = O.compress(Q, K, K, seq_lens=[L], Hq=1, Hkv=1, w=2, k=3)[(0, 0)]
    expect = [1 / 7 + 1 / 8] * 7 + [1 / 8]
    np.testing.assert_allclose(res["scores"], expect, atol=1e-15)
    assert res["idx"].tolist() == [0, 1, 2]


def test_equal_keys_give_uniform_rows_for_any_query():
    L, d = 11, 8
    rng = np.random.default_rng(1)
    K = np.tile(rng.standard_normal((1, 1, d)), (L, 1, 1))
    Q = rng.standard_normal((1, 3, 1, d)) * 5
    res = O.compress(Q, K, K, seq_lens=[L], Hq=1, Hkv=1, w=3, k=2)[(0, 0)]
    expect = [sum(1 / (L - 3 + r + 1) for r in range(3))] * (L - 2) + [1 / (L - 1) + 1 / L, 1 / L]
    np.testing.assert_allclose(res["scores"], expect, atol=1e-14)


@pytest.mark.parametrize("has_decode,alpha", [(False, 0.0), (True, 0.3)])
def test_rows_sum_to_one_and_total_mass(has_decode, alpha):
    rng = np.random.default_rng(2)
    L, d, Hq, Hkv, w = 50, 32, 6, 2, 7
    K = rng.standard_normal((L, Hkv, d))
    Q = rng.standard_normal((1, w + has_decode, Hq, d)) * 3
    pos = O.observation_positions(L, w, has_decode)
    vis = O.visible_mask(pos, L, True)
    P = O.row_probabilities(Q[0, :, 0, :], K[:, 0, :], vis, 1 / math.sqrt(d))
    assert np.all(np.abs(P.sum(axis=1) - 1) <= 1e-12)
    assert np.all(P[~vis] == 0)
    res = O.compress(Q, K, K, seq_lens=[L], Hq=Hq, Hkv=Hkv, w=w, has_decode=has_decode, alpha=alpha, k=5)
    G = Hq // Hkv
    mass = G * (w * (1 - alpha) + alpha) if has_decode else G * w
    for h in range(Hkv):
        assert abs(res[(0, h)]["scores"].sum() - mass) <= 1e-11


# ---------------------------------------------------------------- brute force
def test_matches_full_causal_attention_scipy():
    """Last w rows of full L x L causal softmax attention (scipy)."""
    rng = np.random.default_rng(3)
    L, d, w = 40, 16, 6
    K = rng.standard_normal((L, d))
    Qfull = rng.standard_normal((L, d)) * 2
    logits = Qfull @ K.T / math.sqrt(d)
    logits[np.triu_indices(L, 1)] = -np.inf
    A = scipy.special.softmax(logits, axis=1)
    pos = O.observation_positions(L, w, False)
    P = O.row_probabilities(Qfull[L - w:], K, O.visible_mask(pos, L, True), 1 / math.sqrt(d))
    np.testing.assert_allclose(P, A[L - w:], rtol=0, atol=1e-14)


def test_matches_torch_sdpa_attention_matrix():
    """torch's fp64 scaled-dot-product attention with V = identity returns the
    attention matrix itself; its causal last rows must equal the oracle's."""
    rng = np.random.default_rng(4)
    L, d, w, G = 33, 16, 5, 3
    K = rng.standard_normal((L, 1, d))
    Qfull = rng.standard_normal((G, L, d)) * 2
    A = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qfull)[None], torch.from_numpy(K[:, 0, :])[None, None].expand(1, G, L, d),
        torch.eye(L, dtype=torch.float64)[None, None].expand(1, G, L, L), is_causal=True)[0].numpy()
    Q = Qfull[:, L - w:, :].transpose(1, 0, 2)[None]  # [1, w, G, d]
    S = O.head_scores(Q[0], K, 0, 1, w=w, has_decode=False, alpha=0.0, causal=True, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(S, A[:, L - w:, :].sum(axis=(0, 1)), rtol=0, atol=1e-13)


def test_noncausal_decode_row_sees_whole_prefix():
    rng = np.random.default_rng(5)
    L, d = 20, 8
    K = rng.standard_normal((L, d))
    q = rng.standard_normal((1, d))
    A = scipy.special.softmax(q @ K.T / math.sqrt(d), axis=1)
    pos = O.observation_positions(L, 3, True)
    vis = O.visible_mask(pos, L, True)
    assert vis[-1].all() and pos[-1] == L
    P = O.row_probabilities(q, K, vis[-1:], 1 / math.sqrt(d))
    np.testing.assert_allclose(P, A, atol=1e-15)


# ---------------------------------------------------------------- TideKV's two-pass blockwise form
@pytest.mark.parametrize("block", [1, 3, 16, 64])
def test_blockwise_two_pass_equals_dense(block):
    rng = np.random.default_rng(6)
    L, d, Hq, Hkv, w = 61, 16, 4, 2, 9
    K = rng.standard_normal((L, Hkv, d)) * 2
    Q = rng.standard_normal((w + 1, Hq, d)) * 3
    kw = dict(w=w, has_decode=True, alpha=0.4, causal=True, scale=0.7)
    for h in range(Hkv):
        dense = O.head_scores(Q, K, h, Hkv, **kw)
        blocked = O.blockwise_head_scores(Q, K, h, Hkv, block=block, **kw)
        np.testing.assert_allclose(blocked, dense, rtol=1e-12, atol=1e-15)


def test_blockwise_stats_match_logsumexp():
    rng = np.random.default_rng(7)
    L, d = 100, 8
    K = rng.standard_normal((L, d)) * 4
    q = rng.standard_normal((3, d)) * 4
    vis = O.visible_mask(O.observation_positions(L, 3, False), L, True)
    M, Z = O.blockwise_row_stats(q, K, vis, 1.0, 7)
    logits = np.where(vis, q @ K.T, -np.inf)
    np.testing.assert_allclose(M + np.log(Z), scipy.special.logsumexp(logits, axis=1), rtol=1e-13)


# ---------------------------------------------------------------- pool
@pytest.mark.parametrize("kernel", [1, 3, 5, 7, 9])
def test_pool_matches_torch(kernel):
    rng = np.random.default_rng(kernel)
    S = rng.random(23)
    t = torch.from_numpy(S)[None, None]
    avg = torch.nn.functional.avg_pool1d(t, kernel, stride=1, padding=kernel // 2, count_include_pad=True)
    mx = torch.nn.functional.max_pool1d(t, kernel, stride=1, padding=kernel // 2)
    np.testing.assert_allclose(O.pool1d(S, "avg", kernel), avg[0, 0].numpy(), rtol=1e-15, atol=1e-16)
    np.testing.assert_array_equal(O.pool1d(S, "max", kernel), mx[0, 0].numpy())
    np.testing.assert_array_equal(O.pool1d(S, "none", kernel), S)


def test_pool_short_sequences():
    S = np.array([0.5, 0.25])
    np.testing.assert_allclose(O.pool1d(S, "avg", 7), [0.75 / 7, 0.75 / 7])
    np.testing.assert_array_equal(O.pool1d(S, "max", 7), [0.5, 0.5])
    with pytest.raises(ValueError):
        O.pool1d(S, "avg", 4)


# ---------------------------------------------------------------- top-k
def _brute_topk(P, k):
    """The unique k-subset whose every member beats every non-member
    (higher value, or equal value and lower position)."""
    L = len(P)
    k = min(k, L)
    hits = []
    for sub in itertools.combinations(range(L), k):
        s = set(sub)
        if all(P[i] > P[j] or (P[i] == P[j] and i < j) for i in s for j in range(L) if j not in s):
            hits.append(list(sub))
    assert len(hits) == 1
    return hits[0]


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_exhaustive(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 11))
    P = rng.integers(0, 4, L).astype(float) / 4  # many exact ties
    if seed % 3 == 0:
        P = rng.random(L)
    for k in range(0, L + 2):
        assert O.select_topk(P, k).tolist() == _brute_topk(P, k)


def test_topk_clamps_and_empties():
    P = np.array([3.0, 1.0, 2.0])
    assert O.select_topk(P, 0).tolist() == []
    assert O.select_topk(P, 10).tolist() == [0, 1, 2]


# ---------------------------------------------------------------- gather and plan
def test_gather_is_take():
    rng = np.random.default_rng(8)
    X = rng.standard_normal((30, 3, 4))
    idx = np.array([0, 5, 6, 29])
    np.testing.assert_array_equal(O.gather_rows(X, idx, 2), np.take(X[:, 2, :], idx, axis=0))


def test_plan_offsets_by_hand():
    off = O.plan_offsets([10, 3], 2, [[4, 20], [0, 2]])
    assert off.tolist() == [0, 4, 14, 14, 16]


def test_compress_ragged_consistency():
    rng = np.random.default_rng(9)
    lens = [12, 5, 30]
    Hq, Hkv, d, w = 4, 2, 8, 3
    K = rng.standard_normal((sum(lens), Hkv, d))
    V = rng.standard_normal((sum(lens), Hkv, d))
    Q = rng.standard_normal((3, w, Hq, d))
    budgets = [[4, 12], [9, 0], [1, 30]]
    res = O.compress(Q, K, V, seq_lens=lens, Hq=Hq, Hkv=Hkv, w=w, pool="max", pool_kernel=3, budgets=budgets)
    starts = np.cumsum([0] + lens)
    for b, L in enumerate(lens):
        for h in range(Hkv):
            r = res[(b, h)]
            assert len(r["idx"]) == min(budgets[b][h], L)
            assert np.all(np.diff(r["idx"]) > 0)
            np.testing.assert_array_equal(r["V_out"], V[starts[b] + r["idx"], h])
            # isolated check of this sequence alone
            alone = O.compress(Q[b:b + 1], K[starts[b]:starts[b + 1]], V[starts[b]:starts[b + 1]], seq_lens=[L],
                               Hq=Hq, Hkv=Hkv, w=w, pool="max", pool_kernel=3, budgets=[budgets[b]])
            np.testing.assert_array_equal(alone[(0, h)]["idx"], r["idx"])


def test_rejects_nonfinite():
    K = np.zeros((4, 1, 8))
    K[0, 0, 0] = np.nan
    with pytest.raises(ValueError):
        O.compress(np.zeros((1, 1, 1, 8)), K, K, seq_lens=[4], Hq=1, Hkv=1, w=1, k=1)


# ---------------------------------------------------------------- DeferKV variant: temporal weights, reserved positions
def test_temporal_weights_closed_form():
    # w = 2 prompt rows and a decode row, lambda = ln 2: relative positions -1, 0, 1 weigh 1 : 2 : 4
    np.testing.assert_allclose(O.temporal_row_weights(2, True, np.log(2.0)), [1 / 7, 2 / 7, 4 / 7], rtol=1e-14)
    np.testing.assert_allclose(O.temporal_row_weights(5, False, 0.0), np.full(5, 0.2), rtol=1e-14)
    c = O.temporal_row_weights(32, True, 0.1)
    assert abs(c.sum() - 1.0) < 1e-14
    np.testing.assert_allclose(c[1:] / c[:-1], np.exp(0.1), rtol=1e-12)


def test_temporal_weights_applied_to_rows():
    """Hand keys; prompt row q=+1 at position 7 and decode row q=-1 with
    lambda = ln 3: weights 1/4 and 3/4 of the two rows' probabilities, whose
    values are those of the 8-token worked examples."""
    j = _hand()
    a, b, c = 0.328455, 0.044452, 0.120832  # P of the row q=+1 at position 7
    p_plus = np.array([a, b, b, c, b, b, b, a])
    s_ex3 = np.array([0.352457, 0.221802, 0.221802, 0.186076, 0.221802, 0.221802, 0.221802, 0.352457])
    p_minus = s_ex3 - p_plus  # the row q=-1 (the two rows of the G=2 example sum to s_ex3)
    keys = j["keys_c0"]
    K = np.zeros((8, 1, 128))
    K[:, 0, 0] = keys
    Q = np.zeros((2, 1, 128))
    Q[0, 0, 0] = 1.0
    Q[1, 0, 0] = -1.0
    S = O.head_scores(Q, K, 0, 1, w=1, has_decode=True, alpha=0.0, causal=True, scale=1.0,
                      weighting="exp", lam=np.log(3.0))
    np.testing.assert_allclose(S, 0.25 * p_plus + 0.75 * p_minus, atol=2e-6)


def test_reserved_positions_kept_first():
    a, b, c = 0.328455, 0.044452, 0.120832
    P = np.array([a, b, b, c, b, b, b, a])
    prot = O.protected_mask(8, 1, 2)  # sink {0}, recent {6, 7}
    assert prot.tolist() == [True, False, False, False, False, False, True, True]
    assert O.select_topk(P, 4, prot).tolist() == [0, 3, 6, 7]
    assert O.select_topk(P, 5, prot).tolist() == [0, 1, 3, 6, 7]  # tie among the b's: lowest position
    assert O.select_topk(P, 2, prot).tolist() == [0, 6]  # budget below the reserve: lowest reserved positions
    assert O.select_topk(P, 8, prot).tolist() == list(range(8))
    assert O.protected_mask(3, 5, 5).all()
    assert not O.protected_mask(6, 0, 0).any()


@pytest.mark.parametrize("seed", range(4))
def test_reserve_matches_mask_and_topk(seed):
    """Budget at least the reserve: same as masking the reserved positions out,
    taking the top (k - sink - recent) of the rest and adding the reserve."""
    rng = np.random.default_rng(seed)
    L, sink, recent = 50, 4, 6
    P = rng.random(L)
    for k in (10, 21, 50):
        masked = P.copy()
        masked[:sink] = -np.inf
        masked[L - recent:] = -np.inf
        top = np.argsort(-masked, kind="stable")[:k - sink - recent]
        expect = sorted(set(range(sink)) | set(range(L - recent, L)) | set(top.tolist()))
        assert O.select_topk(P, k, O.protected_mask(L, sink, recent)).tolist() == expect


def test_round_to_bf16_matches_torch_conversion():
    """float32 -> bfloat16 in torch rounds to nearest, ties to even; on values
    that float32 holds exactly the oracle's rounding must agree bit for bit."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000)).astype(np.float32)
    # exact halfway cases between neighbouring bfloat16 values, both parities
    base = torch.randn(4000).to(torch.bfloat16).to(torch.float32).numpy()
    ulp = np.ldexp(1.0, np.frexp(base.astype(np.float64))[1] - 8).astype(np.float32)
    ties = (base.astype(np.float64) + 0.5 * ulp).astype(np.float32)
    sub = (rng.random(2000) * 2.0 ** -126).astype(np.float32)  # bfloat16 subnormal range
    for v in (x, ties, sub, np.array([0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32)):
        want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(O.round_to_bf16(v.astype(np.float64)), want)
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0  # tie, to the even neighbour
    assert O.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_mean_query_matches_torch_bf16_mean():
    """torch's mean over bfloat16 queries (what the DeferKV guide's code runs)
    gives the same rows: the exact mean rounded once to bfloat16."""
    g = torch.Generator().manual_seed(3)
    Q = (torch.randn(9, 32, 128, generator=g) * 11.3).to(torch.bfloat16)
    for h in (0, 3, 7):
        want = Q[:, 4 * h:4 * h + 4, :].mean(dim=1).to(torch.float64).numpy()
        np.testing.assert_array_equal(O.mean_query_rows(Q.to(torch.float64).numpy(), h, 4), want)


def test_mean_query_hand_groups():
    """Hand keys, one window row at position 7, Hq = 4, Hkv = 2.  Group 0 holds
    queries +1 and -1 (mean 0: uniform 1/8 over the 8 visible keys); group 1
    holds +1 and +1 (mean +1: the worked example's row q=+1)."""
    j = _hand()
    a, b, c = 0.328455, 0.044452, 0.120832
    K = np.zeros((8, 2, 128))
    K[:, :, 0] = np.asarray(j["keys_c0"])[:, None]
    Q = np.zeros((1, 4, 128))
    Q[0, :, 0] = [1.0, -1.0, 1.0, 1.0]
    kw = dict(w=1, has_decode=False, alpha=0.0, causal=True, scale=1.0, gqa="mean")
    np.testing.assert_allclose(O.head_scores(Q, K, 0, 2, **kw), np.full(8, 0.125), rtol=1e-14)
    np.testing.assert_allclose(O.head_scores(Q, K, 1, 2, **kw), [a, b, b, c, b, b, b, a], atol=2e-6)


def test_mean_query_equal_heads_is_sum_over_G():
    """When every query head of a group holds the same bfloat16 query, the mean
    is that query, so the mean-query score is the per-head sum divided by G."""
    rng = np.random.default_rng(8)
    L, G, w = 300, 4, 6
    K = rng.standard_normal((L, 1, 128)) / np.sqrt(128)
    q = O.round_to_bf16(rng.standard_normal((w + 1, 1, 128)) * np.sqrt(128))
    Q = np.repeat(q, G, axis=1)
    kw = dict(w=w, has_decode=True, alpha=0.0, causal=True, scale=1.0 / np.sqrt(128), weighting="exp", lam=0.1)
    np.testing.assert_allclose(O.head_scores(Q, K, 0, 1, gqa="mean", **kw),
                               O.head_scores(Q, K, 0, 1, gqa="sum", **kw) / G, rtol=1e-12)


def test_tier_labels_hand():
    """Importance 3, 1, 3, 2, 2, 0 ranks positions 0, 2, 3, 4, 1, 5 (equal
    values: lower position first); two fast and two middle slots."""
    prof = np.array([3.0, 1.0, 3.0, 2.0, 2.0, 0.0])
    assert O.tier_labels(prof, 2, 2).tolist() == [0, 2, 0, 1, 1, 2]
    assert O.tier_labels(prof, 1, 2).tolist() == [0, 2, 1, 1, 2, 2]
    assert O.tier_labels(prof, 0, 3).tolist() == [1, 2, 1, 1, 2, 2]
    assert O.tier_labels(prof, 6, 4).tolist() == [0] * 6
    assert O.tier_labels(prof, 3, 100).tolist() == [0, 1, 0, 0, 1, 1]
    # max pool of width 3: 3, 3, 3, 3, 2, 2 -> positions 0..3 tie at 3
    assert O.tier_labels(prof, 2, 1, "max", 3).tolist() == [0, 0, 1, 2, 2, 2]


@pytest.mark.parametrize("seed", range(3))
def test_tier_labels_invariants(seed):
    """Tier sizes are min(n_fast, L), then min(n_mid, rest); every fast value
    is >= every middle value >= every backing-store value."""
    rng = np.random.default_rng(seed)
    L = 500
    prof = rng.integers(0, 20, L).astype(np.float64)  # many ties
    for nf, nm in ((0, 0), (10, 40), (123, 0), (499, 5), (600, 1)):
        lab = O.tier_labels(prof, nf, nm)
        n0 = min(nf, L)
        n1 = min(nm, L - n0)
        assert (lab == 0).sum() == n0 and (lab == 1).sum() == n1 and (lab == 2).sum() == L - n0 - n1
        for a, b in ((0, 1), (1, 2), (0, 2)):
            if (lab == a).any() and (lab == b).any():
                lo = prof[lab == a].min()
                hi = prof[lab == b].max()
                assert lo >= hi
                # at a tie across the boundary the lower positions sit in the faster tier
                if lo == hi:
                    assert np.nonzero((lab == a) & (prof == lo))[0].max() < np.nonzero((lab == b) & (prof == hi))[0].min()


def test_importance_profile_mass():
    """Each KV head's score sums to G times the row weights' sum (every row is
    a distribution), so a profile over n layers sums to n * Hq * sum(c_r)."""
    rng = np.random.default_rng(4)
    seq_lens = [90, 41]
    Hq, Hkv, w = 8, 2, 5
    layers = []
    for _ in range(3):
        Q = rng.standard_normal((2, w + 1, Hq, 128))
        K = rng.standard_normal((sum(seq_lens), Hkv, 128)) / np.sqrt(128)
        layers.append((Q, K))
    prof = O.importance_profile(layers, seq_lens=seq_lens, Hq=Hq, Hkv=Hkv, w=w, has_decode=True, alpha=0.25)
    for b, L in enumerate(seq_lens):
        assert prof[b].shape == (L,)
        assert abs(prof[b].sum() - 3 * Hq * (w * 0.75 + 0.25)) < 1e-9


def test_importance_profile_hand():
    """Hand keys.  Layer 1: KV head 0 with the query +1 and KV head 1 with the
    query -1, one window row at position 7 (G = 1): together the worked
    example's two-row score.  Layer 2: zero queries, 1/8 per key and head."""
    j = _hand()
    s_ex3 = np.array([0.352457, 0.221802, 0.221802, 0.186076, 0.221802, 0.221802, 0.221802, 0.352457])
    K = np.zeros((8, 2, 128))
    K[:, :, 0] = np.asarray(j["keys_c0"])[:, None]
    Q1 = np.zeros((1, 1, 2, 128))
    Q1[0, 0, 0, 0] = 1.0
    Q1[0, 0, 1, 0] = -1.0
    Q2 = np.zeros((1, 1, 2, 128))
    prof = O.importance_profile([(Q1, K), (Q2, K)], seq_lens=[8], Hq=2, Hkv=2, w=1, scale=1.0)[0]
    np.testing.assert_allclose(prof, s_ex3 + 2 * 0.125, atol=3e-6)


def test_importance_profile_zero_queries():
    """Zero queries make every row uniform over its visible keys: a causal
    window row at position p adds 1/(p+1) to keys 0..p, the decode row 1/L to
    every key; summed over Hq query heads and the layers."""
    L, w, Hq, Hkv = 12, 3, 4, 2
    Q = np.zeros((1, w + 1, Hq, 128))
    K = np.random.default_rng(0).standard_normal((L, Hkv, 128))
    prof = O.importance_profile([(Q, K), (Q, K)], seq_lens=[L], Hq=Hq, Hkv=Hkv, w=w, has_decode=True,
                                alpha=0.5)[0]
    want = np.zeros(L)
    for p in range(L - w, L):
        want[:p + 1] += 0.5 / (p + 1)
    want += 0.5 / L
    np.testing.assert_allclose(prof, 2 * Hq * want, rtol=1e-12)


def test_topk_mass_hand_and_brute_force():
    P = np.array([0.5, 2.0, 1.0, 2.0, 0.25])
    np.testing.assert_array_equal(O.topk_mass(P, [0, 1, 2, 3, 5, 9]), [0.0, 2.0, 4.0, 5.0, 5.75, 5.75])
    rng = np.random.default_rng(2)
    P = rng.random(9)
    for k in range(10):
        best = max((sum(P[list(c)]) for c in itertools.combinations(range(9), k)), default=0.0)
        assert abs(O.topk_mass(P, [k])[0] - best) < 1e-12


def test_greedy_allocate_hand():
    """Sizes 0, 2, 4 (cost = size).  Item 0 gains 5 then 1; item 1 gains 3
    then 3; item 2 gains 1 then 10.  Budget 6: ratios 2.5, 1.5, 0.5 -> item 0
    to size 2; then 0.5, 1.5, 0.5 -> item 1; then 0.5, 1.5, 0.5 -> item 1 to
    size 4; budget spent.  The optimum (item 0 to 2, item 2 to 4: 5 + 11 = 16)
    beats the greedy's 5 + 6 = 11, which pins the greedy rule itself."""
    benefit = [[0, 5, 6], [0, 3, 6], [0, 1, 11]]
    assert O.greedy_allocate(benefit, [0, 2, 4], 6).tolist() == [1, 2, 0]
    assert O.greedy_allocate(benefit, [0, 2, 4], 1).tolist() == [0, 0, 0]  # no step fits
    assert O.greedy_allocate(benefit, [0, 2, 4], 100).tolist() == [2, 2, 2]
    assert O.greedy_allocate(benefit, [1, 2, 4], 2).tolist() == [0, 0, 0]  # smallest sizes over budget
    # equal ratios: the lower item index first
    assert O.greedy_allocate([[0, 4], [0, 4]], [0, 2], 2).tolist() == [1, 0]
    # unequal step costs (sizes 0, 1, 3): item 0's second step adds more (0.7)
    # but at a lower ratio (0.35) than item 1's first step (0.5 per entry)
    assert O.greedy_allocate([[0, 1.0, 1.7], [0, 0.5, 0.6]], [0, 1, 3], 3).tolist() == [1, 1]
    # the best ratio (item 1's second step, 1.5) does not fit the 1 entry left;
    # the best step that fits (item 0's first) is taken instead
    assert O.greedy_allocate([[0, 0.1, 10], [0, 0.5, 5.0]], [0, 1, 4], 2).tolist() == [1, 1]
    # a step that adds nothing is not taken
    assert O.greedy_allocate([[0, 0, 0], [0, 1, 1]], [0, 1, 2], 10).tolist() == [0, 1]


@pytest.mark.parametrize("seed", range(5))
def test_greedy_allocate_optimal_on_concave_uniform_steps(seed):
    """With equal size steps and concave benefits (top-k masses are: each step
    adds the next-largest values), the greedy is the exhaustive optimum."""
    rng = np.random.default_rng(seed)
    sizes = [0, 3, 6, 9, 12]
    items = 4
    benefit = np.stack([O.topk_mass(rng.random(12) ** 3, sizes) for _ in range(items)])
    for total in (0, 5, 9, 17, 30, 48):
        got = O.greedy_allocate(benefit, sizes, total)
        value = sum(benefit[i, got[i]] for i in range(items))
        assert sum(sizes[j] for j in got) <= total
        best = max(sum(benefit[i, c[i]] for i in range(items))
                   for c in itertools.product(range(len(sizes)), repeat=items)
                   if sum(sizes[j] for j in c) <= total)
        assert abs(value - best) < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_streaming_select_equals_whole_prefix_selection(seed):
    """TideKV's blockwise streaming top-k keeps exactly the positions the
    whole-prefix selection keeps (continuous random inputs: no ties), for
    blocks smaller than the pool, ragged last blocks, budgets above the
    length, reserved positions, both weightings and both GQA modes."""
    rng = np.random.default_rng(seed)
    L, Hq, Hkv, w = 157, 8, 2, 6
    K = rng.standard_normal((L, Hkv, 128)) / np.sqrt(128)
    Q = O.round_to_bf16(rng.standard_normal((w + 1, Hq, 128)) * np.sqrt(128) * 0.3)
    pool, kern = [("none", 1), ("avg", 5), ("max", 7), ("avg", 3)][seed]
    kw = dict(w=w, has_decode=True, alpha=0.3, causal=seed != 2, scale=1.0 / np.sqrt(128))
    extra = [dict(), dict(weighting="exp", lam=0.1), dict(gqa="mean"), dict(weighting="exp", lam=1.0, gqa="mean")][seed]
    for h in range(Hkv):
        P = O.pool1d(O.head_scores(Q, K, h, Hkv, **kw, **extra), pool, kern)
        for block, k, sink, recent in ((16, 20, 0, 0), (2, 40, 3, 5), (64, 200, 0, 0), (157, 9, 4, 4), (5, 0, 0, 0)):
            got = O.streaming_select(Q, K, h, Hkv, **kw, **extra, block=block, k=k, pool=pool, pool_kernel=kern,
                                     sink=sink, recent=recent)
            want = O.select_topk(P, k, O.protected_mask(L, sink, recent))
            np.testing.assert_array_equal(got, want)


# ---------------------------------------------------------------- planted mistakes
def _pins_pass():
    """Run the pins above in-process; return False as soon as one fails."""
    checks = [
        lambda: [test_hand_examples(ex) for ex in _hand()["examples"]],
        test_decode_weight_asymmetric,
        test_default_scale_is_inverse_sqrt_d,
        test_consecutive_query_head_grouping,
        test_zero_queries_give_uniform_rows,
        lambda: test_rows_sum_to_one_and_total_mass(True, 0.3),
        test_matches_full_causal_attention_scipy,
        lambda: [test_pool_matches_torch(k) for k in (3, 5)],
        lambda: [test_topk_matches_exhaustive(s) for s in range(6)],
        test_gather_is_take,
        test_temporal_weights_closed_form,
        test_temporal_weights_applied_to_rows,
        test_reserved_positions_kept_first,
        lambda: [test_reserve_matches_mask_and_topk(s) for s in range(2)],
        test_round_to_bf16_matches_torch_conversion,
        test_mean_query_matches_torch_bf16_mean,
        test_mean_query_hand_groups,
        test_mean_query_equal_heads_is_sum_over_G,
        test_tier_labels_hand,
        lambda: [test_tier_labels_invariants(s) for s in range(2)],
        test_importance_profile_mass,
        test_importance_profile_hand,
        test_importance_profile_zero_queries,
        test_topk_mass_hand_and_brute_force,
        test_greedy_allocate_hand,
        lambda: [test_greedy_allocate_optimal_on_concave_uniform_steps(s) for s in range(2)],
        lambda: [test_streaming_select_equals_whole_prefix_selection(s) for s in range(4)],
    ]
    for c in checks:
        try:
            c()
        except AssertionError:
            return False
    return True


def _no_causal(positions, L, causal):
    return np.ones((len(positions), L), dtype=bool)


def _mean_rows(w, has_decode, alpha):
    c = np.ones(w + int(has_decode))
    if has_decode:
        c[:w] = 1 - alpha
        c[w] = alpha
    return c / len(c)


def _swapped_alpha(w, has_decode, alpha):
    c = np.ones(w + int(has_decode))
    if has_decode:
        c[:w] = alpha
        c[w] = 1 - alpha
    return c


def _high_index_ties(P, k, protected=None):
    L = len(P)
    keff = max(0, min(int(k), L))
    prot = np.zeros(L, dtype=bool) if protected is None else np.asarray(protected, dtype=bool)
    order = np.lexsort((-np.arange(L), np.where(prot, 0.0, -P), ~prot))
    return np.sort(order[:keff])


def _unnormalised_temporal(w, has_decode, lam):
    r = np.arange(w, dtype=np.float64) - (w - 1)
    if has_decode:
        r = np.append(r, 1.0)
    return np.exp(lam * r)


def _recent_off_by_one(L, sink, recent):
    keep = np.zeros(L, dtype=bool)
    keep[:max(0, min(int(sink), L))] = True
    if recent > 0:
        keep[max(0, L - int(recent) - 1):L - 1] = True
    return keep


def _bf16_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    _, e = np.frexp(x[nz])
    q = np.maximum(e - 8, -133)
    out[nz] = np.ldexp(np.trunc(np.ldexp(x[nz], -q)), q)
    return out


def _mean_query_unrounded(Q_b, h, G):
    return Q_b[:, h * G:(h + 1) * G, :].mean(axis=1)


def _mean_query_strided(Q_b, h, G):
    Hkv = Q_b.shape[1] // G
    return O.round_to_bf16(Q_b[:, h::Hkv, :].mean(axis=1))


def _tiers_high_index_ties(profile, n_fast, n_mid, pool="none", pool_kernel=1):
    P = O.pool1d(np.asarray(profile, dtype=np.float64), pool, pool_kernel)
    L = len(P)
    order = np.lexsort((-np.arange(L), -P))
    rank = np.empty(L, dtype=np.int64)
    rank[order] = np.arange(L)
    lab = np.full(L, 2, dtype=np.int8)
    lab[rank < n_fast + n_mid] = 1
    lab[rank < n_fast] = 0
    return lab


def _tiers_mid_counts_from_zero(profile, n_fast, n_mid, pool="none", pool_kernel=1):
    P = O.pool1d(np.asarray(profile, dtype=np.float64), pool, pool_kernel)
    L = len(P)
    order = np.lexsort((np.arange(L), -P))
    rank = np.empty(L, dtype=np.int64)
    rank[order] = np.arange(L)
    lab = np.full(L, 2, dtype=np.int8)
    lab[rank < n_mid] = 1  # the middle tier's slots not offset by the fast tier's
    lab[rank < n_fast] = 0
    return lab


def _profile_one_head(layers, *, seq_lens, Hq, Hkv, w, has_decode=False, alpha=0.0, causal=True, scale=None,
                      weighting="alpha", lam=0.0, gqa="sum"):
    starts = np.concatenate([[0], np.cumsum(seq_lens)])
    prof = [np.zeros(int(L)) for L in seq_lens]
    for Q, K in layers:
        sc = (1.0 / np.sqrt(K.shape[2])) if scale is None else scale
        for b in range(len(seq_lens)):
            prof[b] += Hkv * O.head_scores(Q[b], K[starts[b]:starts[b + 1]], 0, Hkv, w=w, has_decode=has_decode,
                                           alpha=alpha, causal=causal, scale=sc, weighting=weighting, lam=lam,
                                           gqa=gqa)
    return prof


def _mass_ascending(P, sizes):
    asc = np.sort(np.asarray(P, dtype=np.float64))
    cum = np.concatenate([[0.0], np.cumsum(asc)])
    return np.array([cum[min(int(k), len(asc))] for k in sizes])


def _greedy_by_benefit_not_ratio(benefit, sizes, total):
    benefit = np.asarray(benefit, dtype=np.float64)
    n = benefit.shape[0]
    choice = np.zeros(n, dtype=np.int64)
    left = int(total) - n * sizes[0]
    if left < 0:
        return choice
    while True:
        best, best_gain = -1, 0.0
        for i in range(n):
            j = choice[i]
            if j + 1 >= len(sizes) or sizes[j + 1] - sizes[j] > left:
                continue
            gain = benefit[i, j + 1] - benefit[i, j]
            if gain > best_gain:
                best, best_gain = i, gain
        if best < 0:
            return choice
        left -= sizes[choice[best] + 1] - sizes[choice[best]]
        choice[best] += 1


def _greedy_stops_at_first_misfit(benefit, sizes, total):
    benefit = np.asarray(benefit, dtype=np.float64)
    n = benefit.shape[0]
    choice = np.zeros(n, dtype=np.int64)
    left = int(total) - n * sizes[0]
    while left >= 0:
        cands = [((benefit[i, choice[i] + 1] - benefit[i, choice[i]]) / (sizes[choice[i] + 1] - sizes[choice[i]]), -i)
                 for i in range(n) if choice[i] + 1 < len(sizes)]
        if not cands:
            break
        r, mi = max(cands)
        i = -mi
        dc = sizes[choice[i] + 1] - sizes[choice[i]]
        if r <= 0 or dc > left:
            break
        left -= dc
        choice[i] += 1
    return choice


def _streaming_no_halo(Q_b, K_b, h, Hkv, *, w, has_decode, alpha, causal, scale, block, k, pool="none",
                       pool_kernel=1, weighting="alpha", lam=0.0, gqa="sum", sink=0, recent=0):
    # each block pooled on its own, zero padded at the block's edges
    L = K_b.shape[0]
    S = O.head_scores(Q_b, K_b, h, Hkv, w=w, has_decode=has_decode, alpha=alpha, causal=causal, scale=scale,
                      weighting=weighting, lam=lam, gqa=gqa)
    P = np.concatenate([O.pool1d(S[s:s + block], pool, pool_kernel) for s in range(0, L, block)])
    return O.select_topk(P, k, O.protected_mask(L, sink, recent))


def _avg_exclude_pad(S, kind, kernel):
    if kind != "avg":
        return O.pool1d.__wrapped__(S, kind, kernel)
    r = (kernel - 1) // 2
    return np.array([S[max(0, i - r):i + r + 1].mean() for i in range(len(S))])


def _off_by_one_window(L, w, has_decode):
    pos = list(range(L - w - 1, L - 1))
    if has_decode:
        pos.append(L)
    return np.asarray(pos)


def _no_max_subtraction_sum_mismatch(q_rows, K_h, vis, scale):
    logits = scale * (q_rows @ K_h.T)
    e = np.where(vis, np.exp(logits), 0.0)
    return e / e.sum()  # normalised over the whole matrix, not per row


def _wrong_gather(X_b, idx, h):
    return X_b[idx, (h + 1) % X_b.shape[1], :].copy()


MUTATIONS = {
    "no_causal_mask": ("visible_mask", _no_causal),
    "mean_not_sum_over_rows": ("row_weights", _mean_rows),
    "alpha_swapped": ("row_weights", _swapped_alpha),
    "ties_to_higher_index": ("select_topk", _high_index_ties),
    "avg_pool_excludes_padding": ("pool1d", _avg_exclude_pad),
    "window_off_by_one": ("observation_positions", _off_by_one_window),
    "softmax_not_per_row": ("row_probabilities", _no_max_subtraction_sum_mismatch),
    "gather_wrong_head": ("gather_rows", _wrong_gather),
    "temporal_weights_unnormalised": ("temporal_row_weights", _unnormalised_temporal),
    "recent_window_off_by_one": ("protected_mask", _recent_off_by_one),
    "bf16_rounding_truncates": ("round_to_bf16", _bf16_truncate),
    "mean_query_not_rounded": ("mean_query_rows", _mean_query_unrounded),
    "mean_query_strided_groups": ("mean_query_rows", _mean_query_strided),
    "tiers_ties_to_higher_index": ("tier_labels", _tiers_high_index_ties),
    "tiers_middle_not_offset": ("tier_labels", _tiers_mid_counts_from_zero),
    "profile_head_0_times_Hkv": ("importance_profile", _profile_one_head),
    "mass_of_smallest_values": ("topk_mass", _mass_ascending),
    "greedy_by_gain_not_ratio": ("greedy_allocate", _greedy_by_benefit_not_ratio),
    "greedy_stops_at_first_misfit": ("greedy_allocate", _greedy_stops_at_first_misfit),
    "streaming_pool_without_halo": ("streaming_select", _streaming_no_halo),
}


def test_pins_pass_unmutated():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    original = getattr(O, attr)
    fn.__wrapped__ = original
    monkeypatch.setattr(O, attr, fn)
    assert not _pins_pass(), f"mutation {name} slipped past every pin"
