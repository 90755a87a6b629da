"""HIP path vs the fp64 oracle, through the C ABI, on an MI355X.

Every segment is compared with the oracle, the full-size workloads' too
(the oracle computes one (sequence, KV head) at a time), besides properties
checked on every segment: exact top-k of the GPU's own pooled scores and
bit-exact gathered rows.
"""

import json
import math
import zlib
import os
import sys

import numpy as np
import pytest
import torch

import oracle.kvsel_oracle as O
import workloads as W
from parity import (Guarded, check_against_oracle, check_scores, check_select_exact, compress_guarded, reserved_mask,
                    segments, to_np64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


@pytest.fixture(scope="module")
def kv():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import attention_token_selection_amd as k

    return k


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(kv, spec, case, with_scores=True):
    """kvsel_compress, then (optionally) kvsel_score on the same workspace,
    every output and the workspace between guard bands (checked)."""
    p = kv.Problem(**W.problem_kwargs(spec))
    Q, K, V = (case[x].to(DEV) for x in "QKV")
    out = compress_guarded(kv, p, Q, K, V, pooled=True)
    scores = None
    if with_scores:
        g = Guarded(DEV)
        scores = g.empty(sum(spec.seq_lens) * spec.Hkv, torch.float32)
        kv.kvsel_score(p, Q, K, scores, out["ws"])
        g.check()
        out["guard"].check()
    torch.cuda.synchronize()
    return p, out, scores


def _oracle(spec, case, heads=None):
    return O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), heads=heads,
                      **W.oracle_kwargs(spec))


# ---------------------------------------------------------------- hand-worked examples
def _hand_examples():
    with open(GOLDEN) as f:
        j = json.load(f)
    return [(j["keys_c0"], ex) for ex in j["examples"]]


@pytest.mark.parametrize("keys,ex", _hand_examples(), ids=lambda v: v["name"] if isinstance(v, dict) else "")
def test_hand_examples(kv, keys, ex):
    _say(f"hand example {ex['name']}")
    case = W.hand_case(keys, ex["q_c0"], ex["Hq"], ex["Hkv"])
    p = kv.Problem(Hq=ex["Hq"], Hkv=ex["Hkv"], w=ex["w"], L=len(keys), has_decode=ex["has_decode"],
                   alpha=ex["alpha"], causal=ex["causal"], scale=1.0, pool=ex["pool"],
                   pool_kernel=ex["pool_kernel"], k=ex["k"])
    out = kv.compress(p, *(case[x].to(DEV) for x in "QKV"))
    torch.cuda.synchronize()
    assert out["idx"].cpu().tolist() == ex["expect_idx"]
    ref = O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), seq_lens=[len(keys)],
                     Hq=ex["Hq"], Hkv=ex["Hkv"], w=ex["w"], has_decode=ex["has_decode"], alpha=ex["alpha"],
                     causal=ex["causal"], scale=1.0, pool=ex["pool"], pool_kernel=ex["pool_kernel"], k=ex["k"])
    st = check_scores(out["pooled"].cpu().numpy(), ref[(0, 0)]["pooled"], rtol=1e-5)
    assert st["max_rel"] < 1e-5


# ---------------------------------------------------------------- small shapes, every segment
@pytest.mark.parametrize("spec", W.small_cases(), ids=lambda s: s.name)
def test_small_parity(kv, spec):
    _say(f"small parity {spec.name} lens={spec.seq_lens[:4]} Hq={spec.Hq} Hkv={spec.Hkv} w={spec.w}")
    case = W.make_case(spec)
    _, out, scores = _run(kv, spec, case)
    ref = _oracle(spec, case)
    st = check_against_oracle(spec, case, out, ref, scores=scores)
    assert st["segments"] == spec.batch * spec.Hkv
    assert st["max_rel"] < 1e-4, st


# ---------------------------------------------------------------- full-size workloads, every segment
@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_config_parity(kv, i):
    spec = W.config(i)
    _say(f"config {i} {spec.name}: generating")
    case = W.make_case(spec, layer=0, device=DEV)
    _say(f"config {i}: running kvsel_compress")
    _, out, scores = _run(kv, spec, case)
    _say(f"config {i}: oracle on all {spec.batch * spec.Hkv} segments")
    case_cpu = {k: v.cpu() for k, v in case.items()}
    ref = _oracle(spec, case_cpu)
    st = check_against_oracle(spec, case_cpu, out, ref, scores=scores)
    _say(f"config {i}: {st}")
    assert st["segments"] == spec.batch * spec.Hkv


@pytest.mark.parametrize("pool,width", [("max", 11), ("avg", 255)])
def test_wide_pool_end_to_end(kv, pool, width):
    """Pools wider than 9 positions take the LDS path of the pool kernel."""
    spec = W.Spec(f"wide_{pool}{width}", [3000, 513], Hq=8, Hkv=2, w=16, pool=pool, pool_kernel=width, k=200,
                  recipe="plant", plant_frac=0.02)
    _say(f"wide pool {spec.name}")
    case = W.make_case(spec)
    _, out, scores = _run(kv, spec, case)
    ref = _oracle(spec, case)
    st = check_against_oracle(spec, case, out, ref, scores=scores)
    assert st["segments"] == spec.batch * spec.Hkv


def test_config2_last_layer(kv):
    spec = W.config(2)
    case = W.make_case(spec, layer=31, device=DEV)
    _, out, _ = _run(kv, spec, case, with_scores=False)
    case_cpu = {k: v.cpu() for k, v in case.items()}
    ref = _oracle(spec, case_cpu)
    st = check_against_oracle(spec, case_cpu, out, ref)
    assert st["segments"] == spec.batch * spec.Hkv


# ---------------------------------------------------------------- entry points compose, determinism
def test_entry_points_compose_and_repeat(kv):
    spec = W.small_cases()[7]  # ragged, per-head budgets
    case = W.make_case(spec)
    p = kv.Problem(**W.problem_kwargs(spec))
    Q, K, V = (case[x].to(DEV) for x in "QKV")
    full = kv.compress(p, Q, K, V)
    again = kv.compress(p, Q, K, V)
    ws, offs = kv.kvsel_plan(p)
    n = sum(spec.seq_lens) * spec.Hkv
    g = Guarded(DEV)
    scores = g.empty(n, torch.float32)
    pooled = g.empty(n, torch.float32)
    idx = g.empty(max(1, offs[-1]), torch.int32)
    Ko = g.empty(max(1, offs[-1]) * 128, torch.bfloat16).view(-1, 128)
    Vo = g.empty(max(1, offs[-1]) * 128, torch.bfloat16).view(-1, 128)
    wsb = g.empty(ws, torch.uint8, fill=0xAB)  # arbitrary initial bytes are fine
    kv.kvsel_score(p, Q, K, scores, wsb)
    kv.kvsel_pool_topk(p, scores, pooled, idx, wsb)
    kv.kvsel_gather(p, idx, K, V, Ko, Vo)
    g.check()
    kept = offs[-1]
    assert torch.equal(full["idx"][:kept], idx[:kept])
    assert torch.equal(again["idx"][:kept], idx[:kept])
    assert torch.equal(full["pooled"], pooled)
    assert torch.equal(again["pooled"], pooled)
    assert torch.equal(full["K_out"][:kept], Ko[:kept])
    assert torch.equal(full["V_out"][:kept], Vo[:kept])


def test_two_passes_equal_score(kv):
    """kvsel_row_stats then kvsel_score_from_stats gives exactly the bytes of
    kvsel_score (the same two passes, launched by the caller)."""
    for i in (3, 5, 11):
        spec = W.small_cases()[i]
        case = W.make_case(spec)
        Q, K = (case[x].to(DEV) for x in "QK")
        n = sum(spec.seq_lens) * spec.Hkv
        g = Guarded(DEV)
        one = g.empty(n, torch.float32)
        two = g.empty(n, torch.float32)
        p = kv.Problem(**W.problem_kwargs(spec))
        ws = g.empty(kv.kvsel_plan(p)[0], torch.uint8)
        kv.kvsel_score(p, Q, K, one, ws)
        kv.kvsel_row_stats(p, Q, K, ws)
        kv.kvsel_score_from_stats(p, Q, K, two, ws)
        g.check()
        assert torch.equal(one, two), spec.name


def test_workspace_shared_across_problems(kv):
    """One workspace serves several different problems in a row."""
    cases = [W.small_cases()[i] for i in (6, 7, 11, 6)]
    big = max(kv.kvsel_plan(kv.Problem(**W.problem_kwargs(s)))[0] for s in cases)
    ws = torch.empty(big, dtype=torch.uint8, device=DEV)
    for spec in cases:
        case = W.make_case(spec)
        p = kv.Problem(**W.problem_kwargs(spec))
        out = kv.alloc_outputs(p, DEV)
        kv.kvsel_compress(p, *(case[x].to(DEV) for x in "QKV"), out["idx"], out["K_out"], out["V_out"],
                          out["pooled"], ws)
        torch.cuda.synchronize()
        ref = _oracle(spec, case)
        check_against_oracle(spec, case, out, ref)


# ---------------------------------------------------------------- selection on given scores (exact)
def _adversarial_scores(kind, L, rng):
    if kind == "integer":
        return rng.integers(0, 50, L).astype(np.float32)
    if kind == "all_equal":
        return np.full(L, 0.25, dtype=np.float32)
    if kind == "two_values":
        return rng.choice(np.array([1.0, 2.0], dtype=np.float32), L)
    if kind == "sorted":
        return np.sort(rng.random(L).astype(np.float32))
    if kind == "reverse":
        return np.sort(rng.random(L).astype(np.float32))[::-1].copy()
    if kind == "tiny_and_zero":
        x = (rng.random(L) < 0.5).astype(np.float32) * np.float32(1e-30)
        return x
    return rng.random(L).astype(np.float32) * np.float32(10.0) ** rng.integers(-20, 2, L).astype(np.float32)


@pytest.mark.parametrize("kind", ["integer", "all_equal", "two_values", "sorted", "reverse", "tiny_and_zero", "spread"])
@pytest.mark.parametrize("pool,kernel", [("none", 1), ("max", 7), ("avg", 5), ("max", 11), ("avg", 255)])
def test_select_exact_on_given_scores(kv, kind, pool, kernel):
    rng = np.random.default_rng(zlib.crc32(f"{kind}/{pool}".encode()))
    lens = [1, 7, 1000, 4099, 70000]
    Hkv = 2
    budgets = [[1, 0], [3, 7], [64, 999], [4099, 1500], [2048, 4096]]
    p = kv.Problem(Hq=2, Hkv=Hkv, w=1, seq_lens=lens, pool=pool, pool_kernel=kernel, budgets=budgets)
    ws, offs = kv.kvsel_plan(p)
    S = np.concatenate([_adversarial_scores(kind, L, rng) for L in lens for _ in range(Hkv)])
    scores = torch.from_numpy(S).to(DEV)
    g = Guarded(DEV)
    pooled = g.empty(scores.numel(), torch.float32)
    idx = g.empty(offs[-1], torch.int32)
    kv.kvsel_pool_topk(p, scores, pooled, idx, g.empty(ws, torch.uint8))
    g.check()
    P = pooled.cpu().numpy()
    I = idx.cpu().numpy()
    spec = W.Spec("given", lens, Hq=2, Hkv=Hkv, pool=pool, pool_kernel=kernel, budgets=budgets)
    for (b, h, L, soff, ooff, keff) in segments(spec, offs):
        seg = S[soff:soff + L]
        if pool == "none":
            np.testing.assert_array_equal(P[soff:soff + L], seg)
        elif pool == "max":
            np.testing.assert_array_equal(P[soff:soff + L], O.pool1d(seg.astype(np.float64), "max", kernel))
        else:
            # fp32 window sums of up to 255 terms: allow their rounding
            check_scores(P[soff:soff + L], O.pool1d(seg.astype(np.float64), "avg", kernel),
                         rtol=1e-6 if kernel <= 9 else 2e-5)
        check_select_exact(I[ooff:ooff + keff], P[soff:soff + L], keff)


@pytest.mark.parametrize("kind", ["two_values", "all_equal", "spread", "reverse"])
@pytest.mark.parametrize("sink,recent", [(16, 32), (0, 100), (5000, 0), (3, 70000), (2047, 2049)])
def test_select_reserved_on_given_scores(kv, kind, sink, recent):
    """Reserved sink/recent positions are kept first, then the highest scores;
    budgets below, at and above the reserved count."""
    rng = np.random.default_rng(zlib.crc32(f"{kind}/{sink}/{recent}".encode()))
    lens = [1, 7, 1000, 4099, 70000]
    Hkv = 2
    budgets = [[1, 0], [3, 7], [40, 999], [4099, 3000], [2048, 6000]]
    p = kv.Problem(Hq=2, Hkv=Hkv, w=1, seq_lens=lens, pool="max", pool_kernel=7, budgets=budgets, sink=sink,
                   recent=recent)
    ws, offs = kv.kvsel_plan(p)
    S = np.concatenate([_adversarial_scores(kind, L, rng) for L in lens for _ in range(Hkv)])
    scores = torch.from_numpy(S).to(DEV)
    g = Guarded(DEV)
    pooled = g.empty(scores.numel(), torch.float32)
    idx = g.empty(offs[-1], torch.int32)
    kv.kvsel_pool_topk(p, scores, pooled, idx, g.empty(ws, torch.uint8))
    g.check()
    P = pooled.cpu().numpy()
    I = idx.cpu().numpy()
    spec = W.Spec("given", lens, Hq=2, Hkv=Hkv, pool="max", pool_kernel=7, budgets=budgets)
    for (b, h, L, soff, ooff, keff) in segments(spec, offs):
        # the pooled output holds the real pooled values, reserved or not
        np.testing.assert_array_equal(P[soff:soff + L], O.pool1d(S[soff:soff + L].astype(np.float64), "max", 7))
        res = reserved_mask(L, sink, recent)
        check_select_exact(I[ooff:ooff + keff], P[soff:soff + L], keff, where=f"segment {(b, h)}", reserved=res)
        # and the oracle's own selection rule agrees exactly on these fp32 values
        ref = O.select_topk(P[soff:soff + L].astype(np.float64), keff, O.protected_mask(L, sink, recent))
        np.testing.assert_array_equal(I[ooff:ooff + keff], ref)


@pytest.mark.parametrize("make", [W.deferkv_full, W.deferkv_guide_full], ids=["sum", "mean_query"])
def test_deferkv_full_size(kv, make):
    """The guide's defaults on a 32K-key layer: exp weights (lambda 0.1) over
    32 prompt rows and the decode row, 16 sinks and 32 recent kept; with the
    per-head sum, and with the guide's mean query per group."""
    spec = make()
    _say(f"{spec.name}: generating")
    case = W.make_case(spec, layer=0, device=DEV)
    _, out, scores = _run(kv, spec, case)
    _say(f"{spec.name}: oracle on every segment")
    case_cpu = {k: v.cpu() for k, v in case.items()}
    ref = _oracle(spec, case_cpu)
    st = check_against_oracle(spec, case_cpu, out, ref, scores=scores)
    _say(f"{spec.name}: {st}")
    assert st["segments"] == spec.batch * spec.Hkv


def test_exp_weights_closed_forms(kv):
    """lambda = 0 weights every row 1/w' (so w' times the scores equal the
    unweighted sum); a very large lambda leaves only the newest row."""
    base = dict(Hq=8, Hkv=2, w=8, seq_lens=[900, 300], causal=True, pool="none", k=0)
    spec = W.Spec("exp_closed", [900, 300], Hq=8, Hkv=2, w=8, has_decode=True, recipe="decode_corr")
    case = W.make_case(spec)
    Q, K = (case[x].to(DEV) for x in "QK")
    n = sum(spec.seq_lens) * spec.Hkv

    def score(**kw):
        p = kv.Problem(**base, **kw)
        ws, _ = kv.kvsel_plan(p)
        g = Guarded(DEV)
        out = g.empty(n, torch.float32)
        kv.kvsel_score(p, Q, K, out, g.empty(ws, torch.uint8))
        g.check()
        return out.cpu().numpy().astype(np.float64)

    # prompt rows only: there the alpha weighting gives every row weight 1
    Qp = Q[:, :8].contiguous()
    p_alpha = kv.Problem(**base)
    p_exp0 = kv.Problem(**base, weighting="exp", lam=0.0)
    ws, _ = kv.kvsel_plan(p_alpha)
    g = Guarded(DEV)
    a = g.empty(n, torch.float32)
    e = g.empty(n, torch.float32)
    wsb = g.empty(ws, torch.uint8)
    kv.kvsel_score(p_alpha, Qp, K, a, wsb)
    kv.kvsel_score(p_exp0, Qp, K, e, wsb)
    g.check()
    check_scores(8.0 * e.cpu().numpy().astype(np.float64), a.cpu().numpy().astype(np.float64), "lambda=0")
    # lambda huge: the decode row alone, which is alpha = 1
    big = score(has_decode=True, weighting="exp", lam=1000.0)
    dec = score(has_decode=True, alpha=1.0)
    check_scores(big, dec, "lambda=1000")


# ---------------------------------------------------------------- gather on given indices
def test_gather_given_indices(kv):
    rng = np.random.default_rng(11)
    lens = [33, 1000, 5]
    Hkv = 4
    budgets = [[5, 33, 0, 1], [100, 7, 999, 1000], [5, 2, 1, 3]]
    p = kv.Problem(Hq=4, Hkv=Hkv, w=1, seq_lens=lens, budgets=budgets)
    _, offs = kv.kvsel_plan(p)
    K = torch.randn(sum(lens), Hkv, 128).to(torch.bfloat16)
    V = torch.randn(sum(lens), Hkv, 128).to(torch.bfloat16)
    idx = np.zeros(offs[-1], dtype=np.int32)
    spec = W.Spec("given", lens, Hq=4, Hkv=Hkv, budgets=budgets)
    for (b, h, L, soff, ooff, keff) in segments(spec, offs):
        idx[ooff:ooff + keff] = rng.integers(-3, L + 3, keff)  # includes out-of-range entries
    g = Guarded(DEV)
    Ko = g.empty(offs[-1] * 128, torch.bfloat16, fill=7).view(-1, 128)
    Vo = g.empty(offs[-1] * 128, torch.bfloat16, fill=7).view(-1, 128)
    kv.kvsel_gather(p, torch.from_numpy(idx).to(DEV), K.to(DEV), V.to(DEV), Ko, Vo)
    g.check()
    Ko, Vo = Ko.cpu(), Vo.cpu()
    starts = np.concatenate([[0], np.cumsum(lens)])
    for (b, h, L, soff, ooff, keff) in segments(spec, offs):
        for j in range(keff):
            pos = int(idx[ooff + j])
            if 0 <= pos < L:
                assert torch.equal(Ko[ooff + j], K[starts[b] + pos, h])
                assert torch.equal(Vo[ooff + j], V[starts[b] + pos, h])
            else:
                assert not Ko[ooff + j].any() and not Vo[ooff + j].any()


# ---------------------------------------------------------------- graph capture and replay
def test_graph_replays_match_eager(kv):
    """Capture kvsel_compress for two layers, replay several times with eager
    library work and synchronisations in between; every replay must equal the
    eager result bit for bit."""
    spec = W.small_cases()[6]
    p = kv.Problem(**W.problem_kwargs(spec))
    cases = [{k: v.to(DEV) for k, v in W.make_case(spec, layer=l).items()} for l in range(3)]
    eager = [kv.compress(p, c["Q"], c["K"], c["V"]) for c in cases[:2]]
    torch.cuda.synchronize()
    ws = torch.empty(kv.kvsel_plan(p)[0], dtype=torch.uint8, device=DEV)
    outs = [kv.alloc_outputs(p, DEV) for _ in range(2)]
    stream = torch.cuda.Stream(device=DEV)
    calls = [kv.bind_compress(p, c["Q"], c["K"], c["V"], o["idx"], o["K_out"], o["V_out"], o["pooled"], ws, stream)
             for c, o in zip(cases, outs)]
    with torch.cuda.stream(stream):
        for call in calls:
            call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for call in calls:
            call()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:  # poison the outputs
            o["idx"].fill_(-7)
            o["K_out"].fill_(3.0)
            o["pooled"].fill_(-1.0)
        kv.compress(p, cases[2]["Q"], cases[2]["K"], cases[2]["V"])  # eager work on the same library
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e["idx"], o["idx"]), f"replay {rep}: idx"
            assert torch.equal(e["K_out"], o["K_out"]), f"replay {rep}: K_out"
            assert torch.equal(e["V_out"], o["V_out"]), f"replay {rep}: V_out"
            assert torch.equal(e["pooled"], o["pooled"]), f"replay {rep}: pooled"


# ---------------------------------------------------------------- the longest supported sequence
def test_longest_sequence(kv):
    """One sequence of 2^20 keys (the documented limit: 512 selection chunks)
    at the Llama-3.1-8B shape, k = 4096: exact selection and gather on every
    head, and one head against the oracle (which scores that head alone)."""
    L = 1 << 20
    spec = W.Spec("longest_L1M_max7_k4096", [L], w=32, pool="max", pool_kernel=7, k=4096, recipe="plant",
                  plant_frac=0.002)
    _say(f"{spec.name}: generating")
    case = W.make_case(spec, layer=0, device=DEV)
    p = kv.Problem(**W.problem_kwargs(spec))
    out = kv.compress(p, case["Q"], case["K"], case["V"])
    torch.cuda.synchronize()
    idx = out["idx"]
    offs = out["out_offsets"]
    pooled = out["pooled"].cpu().numpy()
    for h in range(spec.Hkv):
        seg = idx[offs[h]:offs[h + 1]].long()
        assert torch.equal(out["K_out"][offs[h]:offs[h + 1]], case["K"][seg, h])
        assert torch.equal(out["V_out"][offs[h]:offs[h + 1]], case["V"][seg, h])
        check_select_exact(seg.cpu().numpy(), pooled[h * L:(h + 1) * L], offs[h + 1] - offs[h], where=f"head {h}")
    h = 5
    G = spec.Hq // spec.Hkv
    _say(f"{spec.name}: oracle on head {h}")
    Qg = to_np64(case["Q"][0, :, h * G:(h + 1) * G])
    Kh = to_np64(case["K"][:, h:h + 1])
    S = O.head_scores(Qg, Kh, 0, 1, w=spec.w, has_decode=False, alpha=0.0, causal=True, scale=1.0 / math.sqrt(128))
    P = O.pool1d(S, "max", 7)
    ref_idx = O.select_topk(P, spec.k)
    st = check_scores(pooled[h * L:(h + 1) * L], P, f"pooled head {h}")
    from parity import check_selection
    d = check_selection(idx[offs[h]:offs[h + 1]].cpu().numpy(), ref_idx, P, spec.k, L)
    _say(f"{spec.name}: head {h} max_rel {st['max_rel']:.2e}, near-tie differences {d}")
