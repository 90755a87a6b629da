"""TideKV's memory-bounded streaming form of kvsel_compress (stream_keys > 0)
on an MI355X, through the C ABI: against the fp64 oracle, and against the
whole-prefix form of the same call."""

import sys

import numpy as np
import pytest
import torch

import oracle.kvsel_oracle as O
import workloads as W
from parity import check_against_oracle, compress_guarded, kth_value, reserved_mask, segments, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def kv():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import attention_token_selection_amd as k

    return k


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _streamed(kv, spec, case, C):
    p = kv.Problem(**W.problem_kwargs(spec), stream_keys=C)
    out = compress_guarded(kv, p, *(case[x].to(DEV) for x in "QKV"), pooled=False)
    torch.cuda.synchronize()
    return out


def _whole(kv, spec, case):
    p = kv.Problem(**W.problem_kwargs(spec))
    out = compress_guarded(kv, p, *(case[x].to(DEV) for x in "QKV"), pooled=True)
    torch.cuda.synchronize()
    return out


def _check_same_as_whole(spec, s_out, w_out, rtol=1e-5):
    """Same kept sets as the whole-prefix form, except positions whose pooled
    score lies within rtol of that segment's k-th value."""
    si = s_out["idx"].cpu().numpy()
    wi = w_out["idx"].cpu().numpy()
    P = w_out["pooled"].cpu().numpy().astype(np.float64)
    assert s_out["out_offsets"] == w_out["out_offsets"]
    diffs = 0
    for (b, h, L, soff, ooff, keff) in segments(spec, w_out["out_offsets"]):
        a = si[ooff:ooff + keff]
        c = wi[ooff:ooff + keff]
        assert np.all(np.diff(a) > 0)
        d = np.setxor1d(a, c)
        if len(d):
            res = reserved_mask(L, spec.sink, spec.recent)
            assert not res[d].any()
            seg = P[soff:soff + L]
            tau = kth_value(seg[~res], keff - int(res.sum()))
            assert np.all(np.abs(seg[d] - tau) <= rtol * tau), (b, h, d[:8], seg[d][:8], tau)
        diffs += len(d)
    return diffs


STREAM_CASES = [
    (W.Spec("st_plain", [9000], Hq=8, Hkv=2, w=16, pool="max", pool_kernel=7, k=300, recipe="plant"), 2048),
    (W.Spec("st_ragged", [5000, 700, 12289], Hq=16, Hkv=4, w=12, pool="avg", pool_kernel=5,
            budgets=[[0, 40, 5000, 4096], [700, 1, 30, 2000], [64, 3000, 12289, 129]], recipe="plant",
            plant_frac=0.03), 2048),
    (W.Spec("st_deferkv", [7000], Hq=32, Hkv=8, w=32, has_decode=True, pool="max", pool_kernel=7, k=500,
            weighting="exp", lam=0.1, sink=16, recent=32, recipe="decode_corr"), 2048),
    (W.Spec("st_meanq_nocausal", [6000], Hq=32, Hkv=8, w=20, has_decode=True, alpha=0.5, causal=False,
            pool="none", k=100, gqa="mean", recipe="decode_corr"), 2048),
    (W.Spec("st_wide_pool", [4500], Hq=8, Hkv=2, w=8, pool="avg", pool_kernel=255, k=600, recipe="plant"), 2048),
    (W.Spec("st_reserve_over", [3000], Hq=8, Hkv=2, w=8, pool="max", pool_kernel=3, budgets=[[20, 3000]],
            sink=10, recent=2100, recipe="plain"), 2048),
    # running rows of 4096 < kslot + C <= 8192 slots (eight per thread of the selection)
    (W.Spec("st_rows8", [9000], Hq=8, Hkv=2, w=16, pool="avg", pool_kernel=9, k=3000, recipe="zipf"), 4096),
    # every score equal (logits scaled to nothing, no mask): the threshold bin holds every
    # key, so the running selection takes its radix rounds; ties go to the lower position
    (W.Spec("st_ties", [6000], Hq=8, Hkv=2, w=8, causal=False, scale=1e-30, pool="max", pool_kernel=3, k=700,
            recipe="plain"), 2048),
    # a running row longer than the fused selection takes (the step-wise path)
    (W.Spec("st_long_row", [3000], Hq=8, Hkv=2, w=8, pool="max", pool_kernel=5, k=100, recipe="plant"), 32768),
]


@pytest.mark.parametrize("spec,C", STREAM_CASES, ids=[s.name for s, _ in STREAM_CASES])
def test_streaming_small(kv, spec, C):
    _say(f"streaming {spec.name} lens={spec.seq_lens} C={C}")
    case = W.make_case(spec)
    s_out = _streamed(kv, spec, case, C)
    ref = O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), **W.oracle_kwargs(spec))
    st = check_against_oracle(spec, case, {**s_out, "pooled": None}, ref)
    assert st["segments"] == spec.batch * spec.Hkv
    d = _check_same_as_whole(spec, s_out, _whole(kv, spec, case))
    _say(f"streaming {spec.name}: oracle near-ties {st['near_tie_diffs']}, differs from whole-prefix at {d}")


def test_streaming_full_size(kv):
    """The Llama-3.1-8B-shaped 32K-key layer in four steps of 8192 keys."""
    spec = W.config(2)
    case = W.make_case(spec, layer=0, device=DEV)
    s_out = _streamed(kv, spec, case, 8192)
    d = _check_same_as_whole(spec, s_out, _whole(kv, spec, case))
    case_cpu = {k: v.cpu() for k, v in case.items()}
    ref = O.compress(to_np64(case_cpu["Q"]), to_np64(case_cpu["K"]), to_np64(case_cpu["V"]),
                     **W.oracle_kwargs(spec))
    st = check_against_oracle(spec, case_cpu, {**s_out, "pooled": None}, ref)
    _say(f"streaming full size: differs from whole-prefix at {d}; oracle {st}")
    assert st["segments"] == spec.batch * spec.Hkv


def test_streaming_graph_replays_match_eager(kv):
    """The fused streaming form (two alternating key rows per segment, one
    selection launch per step) captured into a graph for two layers and
    replayed several times, with eager library work and synchronisations in
    between: every replay must equal the eager result bit for bit."""
    spec = W.Spec("st_graph", [20000], Hq=32, Hkv=8, w=32, pool="max", pool_kernel=7, k=700, recipe="runs",
                  plant_frac=0.01)
    p = kv.Problem(**W.problem_kwargs(spec), stream_keys=4096)
    cases = [{k: v.to(DEV) for k, v in W.make_case(spec, layer=l).items()} for l in range(3)]
    stream = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(stream):
        eager = [kv.compress(p, c["Q"], c["K"], c["V"], pooled=False, stream=stream) for c in cases[:2]]
    torch.cuda.synchronize()
    ws = torch.empty(kv.kvsel_plan(p)[0], dtype=torch.uint8, device=DEV)
    outs = [kv.alloc_outputs(p, DEV, pooled=False) for _ in range(2)]
    calls = [kv.bind_compress(p, c["Q"], c["K"], c["V"], o["idx"], o["K_out"], o["V_out"], None, ws, stream)
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
        kv.compress(p, cases[2]["Q"], cases[2]["K"], cases[2]["V"], pooled=False)  # eager work on the library
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            assert torch.equal(e["idx"], o["idx"]), f"replay {rep}: idx"
            assert torch.equal(e["K_out"], o["K_out"]), f"replay {rep}: K_out"
            assert torch.equal(e["V_out"], o["V_out"]), f"replay {rep}: V_out"
