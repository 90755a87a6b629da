"""Adaptive budgets on an MI355X, through the C ABI: the kept importance of
candidate budgets (kvsel_topk_mass), KVDrive's greedy allocation over
(layer, head) pairs (kvsel_allocate_budgets, host), and compression with the
allocated per-head budgets, against the fp64 oracle."""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle.kvsel_oracle as O
import workloads as W
from parity import Guarded, check_against_oracle, check_scores, compress_guarded, segments, to_np64

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


def _mass(kv, p, pooled, sizes):
    ws_bytes, _ = kv.kvsel_plan(p)
    g = Guarded(DEV)
    ws = g.empty(ws_bytes, torch.uint8)
    mass = g.empty(p.batch * p.Hkv * len(sizes), torch.float32, fill=float("nan"))
    kv.kvsel_topk_mass(p, pooled, sizes, mass, ws)
    g.check()
    return mass.cpu().numpy().reshape(p.batch * p.Hkv, len(sizes))


@pytest.mark.parametrize("kind", ["spread", "ties"])
def test_topk_mass_on_given_scores(kv, kind):
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    lens = [1, 50, 3000, 70000]
    Hkv = 2
    p = kv.Problem(Hq=2, Hkv=Hkv, w=1, seq_lens=lens, k=0)
    if kind == "ties":
        S = rng.integers(0, 8, sum(lens) * Hkv).astype(np.float32)
    else:
        S = (rng.random(sum(lens) * Hkv) * 10.0 ** rng.integers(-6, 2, sum(lens) * Hkv)).astype(np.float32)
    sizes = [0, 1, 49, 2048, 5000, 100000]
    got = _mass(kv, p, torch.from_numpy(S).to(DEV), sizes)
    spec = W.Spec("given", lens, Hq=2, Hkv=Hkv)
    for si, (b, h, L, soff, _, _) in enumerate(segments(spec, [0] * (len(lens) * Hkv + 1))):
        want = O.topk_mass(S[soff:soff + L].astype(np.float64), sizes)
        np.testing.assert_allclose(got[si], want, rtol=1e-5, atol=0, err_msg=f"segment {(b, h)}")


def test_adaptive_budgets_end_to_end(kv):
    """Two layers of a ragged batch: pooled scores, their kept importance for
    five candidate budgets, the greedy allocation of 200 entries per pair on
    average, then compression of each layer with its allocated budgets."""
    spec = W.Spec("adaptive", [900, 2500], Hq=16, Hkv=4, w=16, pool="max", pool_kernel=5, k=0, recipe="plant",
                  plant_frac=0.03)
    sizes = [32, 64, 128, 256, 512]
    p = kv.Problem(**W.problem_kwargs(spec))
    cases = [W.make_case(spec, layer=l) for l in range(2)]
    benefit = []
    for case in cases:
        out = compress_guarded(kv, p, *(case[x].to(DEV) for x in "QKV"))
        torch.cuda.synchronize()
        m = _mass(kv, p, out["pooled"], sizes)
        ref = O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), **W.oracle_kwargs(spec))
        gp = out["pooled"].cpu().numpy()
        for si, (b, h, L, soff, _, _) in enumerate(segments(spec, out["out_offsets"])):
            np.testing.assert_allclose(m[si], O.topk_mass(gp[soff:soff + L].astype(np.float64), sizes), rtol=1e-5)
            check_scores(m[si], O.topk_mass(ref[(b, h)]["pooled"], sizes), f"mass {(b, h)}")
        benefit.append(m.astype(np.float64))
    benefit = np.concatenate(benefit)  # items: layer-major, then (sequence, head)
    total = 200 * benefit.shape[0]
    budgets = kv.kvsel_allocate_budgets(benefit, sizes, total)
    np.testing.assert_array_equal(budgets, np.asarray(sizes)[O.greedy_allocate(benefit, sizes, total)])
    assert budgets.sum() <= total and len(set(budgets.tolist())) > 1
    per = spec.batch * spec.Hkv
    for l, case in enumerate(cases):
        bl = budgets[l * per:(l + 1) * per].reshape(spec.batch, spec.Hkv).tolist()
        s2 = W.Spec(**{**spec.__dict__, "budgets": bl})
        p2 = kv.Problem(**W.problem_kwargs(s2))
        out = compress_guarded(kv, p2, *(case[x].to(DEV) for x in "QKV"))
        torch.cuda.synchronize()
        ref = O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), **W.oracle_kwargs(s2))
        st = check_against_oracle(s2, case, out, ref)
        assert st["segments"] == per


def test_topk_mass_full_size(kv):
    """One layer of the Llama-3.1-8B-shaped 32K-key workload, all 8 heads."""
    spec = W.config(2)
    case = W.make_case(spec, layer=0, device=DEV)
    p = kv.Problem(**W.problem_kwargs(spec))
    out = compress_guarded(kv, p, case["Q"], case["K"], case["V"])
    sizes = [256, 512, 1024, 2048, 4096]
    m = _mass(kv, p, out["pooled"], sizes)
    gp = out["pooled"].cpu().numpy()
    for si, (b, h, L, soff, _, _) in enumerate(segments(spec, out["out_offsets"])):
        np.testing.assert_allclose(m[si], O.topk_mass(gp[soff:soff + L].astype(np.float64), sizes), rtol=1e-5)
    _say(f"full-size kept importance, head 0: {m[0].tolist()}")
