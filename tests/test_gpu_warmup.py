"""KVDrive's importance-guided warm-up on an MI355X, through the C ABI:
the per-position importance profile summed over KV heads and layers
(kvsel_profile_layer), and the three-tier ranking (kvsel_tier_rank), against
the fp64 oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle.kvsel_oracle as O
import workloads as W
from parity import RTOL, Guarded, check_finite, check_scores, to_np64

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


def _profile(kv, spec, n_layers, pool="none", pool_kernel=1):
    kw = W.problem_kwargs(spec)
    kw.update(pool=pool, pool_kernel=pool_kernel)
    p = kv.Problem(**kw)
    ws_bytes, _ = kv.kvsel_plan(p)
    g = Guarded(DEV)
    ws = g.empty(ws_bytes, torch.uint8)
    prof = g.empty(sum(spec.seq_lens), torch.float32, fill=float("nan"))  # every value must be written
    layers = []
    for layer in range(n_layers):
        case = W.make_case(spec, layer=layer, device=DEV)
        kv.kvsel_profile_layer(p, case["Q"], case["K"], prof, ws, accumulate=layer > 0)
        layers.append((to_np64(case["Q"]), to_np64(case["K"])))
    g.check()
    return p, ws, prof, layers


def _oracle_profile(spec, layers):
    return O.importance_profile(layers, seq_lens=spec.seq_lens, Hq=spec.Hq, Hkv=spec.Hkv, w=spec.w,
                                has_decode=spec.has_decode, alpha=spec.alpha, causal=spec.causal,
                                scale=(spec.scale if spec.scale else None), weighting=spec.weighting, lam=spec.lam,
                                gqa=spec.gqa)


def _tiers(kv, p, ws, prof, n_fast, n_mid):
    g = Guarded(DEV)
    tier = g.empty(prof.numel(), torch.int8, fill=7)
    kv.kvsel_tier_rank(p, prof, n_fast, n_mid, tier, ws)
    g.check()
    return tier.cpu().numpy()


def _check_tiers(spec, gpu_prof, gpu_tier, ref_prof, n_fast, n_mid, pool, kernel):
    """Exact against the oracle's ranking of the GPU's own fp32 profile (max
    and no pool are exact in fp32); against the oracle's profile, labels may
    differ only at positions whose value is within RTOL of a tier boundary."""
    off = np.concatenate([[0], np.cumsum(spec.seq_lens)])
    diffs = 0
    for b, L in enumerate(spec.seq_lens):
        g = gpu_tier[off[b]:off[b + 1]]
        assert set(np.unique(g).tolist()) <= {0, 1, 2}
        mine = gpu_prof[off[b]:off[b + 1]].astype(np.float64)
        if pool != "avg":
            np.testing.assert_array_equal(g, O.tier_labels(mine, n_fast, n_mid, pool, kernel),
                                          err_msg=f"sequence {b}: ranking of the GPU profile")
        ref = O.tier_labels(ref_prof[b], n_fast, n_mid, pool, kernel)
        P = O.pool1d(ref_prof[b], pool, kernel)
        srt = np.sort(P)[::-1]
        bounds = [srt[min(n, L) - 1] for n in (n_fast, n_fast + n_mid) if 0 < n < L]
        bad = np.nonzero(g != ref)[0]
        for i in bad:
            assert any(abs(P[i] - t) <= RTOL * t for t in bounds), (b, int(i), P[i], bounds)
        diffs += len(bad)
    return diffs


@pytest.mark.parametrize("pool,kernel", [("none", 1), ("max", 5), ("avg", 7)])
def test_warmup_small(kv, pool, kernel):
    spec = W.Spec("warm_small", [700, 1500, 37], Hq=16, Hkv=4, w=16, has_decode=True, alpha=0.4,
                  recipe="plant", plant_frac=0.03)
    _say(f"warm-up small, pool {pool} {kernel}")
    p, ws, prof, layers = _profile(kv, spec, 3, pool, kernel)
    gp = prof.cpu().numpy()
    check_finite(gp, "profile")
    ref = _oracle_profile(spec, layers)
    off = np.concatenate([[0], np.cumsum(spec.seq_lens)])
    for b in range(spec.batch):
        check_scores(gp[off[b]:off[b + 1]], ref[b], f"profile of sequence {b}")
    for n_fast, n_mid in ((100, 300), (0, 50), (40, 0), (2000, 10), (0, 0)):
        g = _tiers(kv, p, ws, prof, n_fast, n_mid)
        _check_tiers(spec, gp, g, ref, n_fast, n_mid, pool, kernel)


def test_warmup_mean_query_exp(kv):
    """The profile follows the problem's weighting and grouped-query mode."""
    spec = W.Spec("warm_meanq", [1200], Hq=32, Hkv=8, w=32, has_decode=True, weighting="exp", lam=0.1,
                  gqa="mean", recipe="decode_corr")
    p, ws, prof, layers = _profile(kv, spec, 2)
    ref = _oracle_profile(spec, layers)
    check_scores(prof.cpu().numpy(), ref[0], "profile")


def test_warmup_full_size(kv):
    """Four layers of the Llama-3.1-8B-shaped 32K-key workload; 2048 fast and
    8192 middle slots."""
    spec = W.config(2)
    _say("warm-up full size: profiling 4 layers")
    p, ws, prof, layers = _profile(kv, spec, 4)
    _say("warm-up full size: oracle")
    ref = _oracle_profile(spec, layers)
    gp = prof.cpu().numpy()
    st = check_scores(gp, ref[0], "profile")
    g = _tiers(kv, p, ws, prof, 2048, 8192)
    d = _check_tiers(spec, gp, g, ref, 2048, 8192, "none", 1)
    _say(f"warm-up full size: max_rel {st['max_rel']:.2e}, boundary ties {d}")
    assert (g == 0).sum() == 2048 and (g == 1).sum() == 8192
