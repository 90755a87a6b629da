"""The resident scoring path of kvsel_compress on an MI355X.

kvsel_compress scores a problem with one fused launch when it fits (at most
256 observation rows per KV head, pools at most 33 wide, key blocks of 512
within the caller's key_chunk).  These tests pin what is particular to it:

* a block that stops waiting for its segment and computes the missing
  blocks' statistics itself (forced from the host with KVSEL_SPIN_CAP=0)
  gives exactly the bytes of the normal path;
* the two-launch scoring (KVSEL_FORCE_TWO_PASS=1) still matches the oracle
  through kvsel_compress, and agrees with the resident path;
* shapes at the path's edges: one key, a block of exactly 512, 513 keys, a
  33-wide pool, 256 rows.
"""

import os
import sys

import numpy as np
import pytest
import torch

import oracle.kvsel_oracle as O
import workloads as W
from parity import check_against_oracle, check_scores, check_selection, segments, to_np64

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


class _env:
    """Sets environment variables for the calls inside the block."""

    def __init__(self, **kw):
        self.kw = kw

    def __enter__(self):
        self.old = {k: os.environ.get(k) for k in self.kw}
        os.environ.update({k: str(v) for k, v in self.kw.items()})

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _compress(kv, spec, case):
    p = kv.Problem(**W.problem_kwargs(spec))
    out = kv.compress(p, *(case[x].to(DEV) for x in "QKV"), pooled=True)
    torch.cuda.synchronize()
    return out


EDGE = [
    W.Spec("r_L1", [1], Hq=4, Hkv=1, w=1, pool="avg", pool_kernel=5, k=1, recipe="plain"),
    W.Spec("r_L512", [512], Hq=32, Hkv=8, w=32, pool="max", pool_kernel=7, k=100, recipe="plant"),
    W.Spec("r_L513", [513], Hq=32, Hkv=8, w=32, pool="avg", pool_kernel=7, k=100, recipe="plant"),
    W.Spec("r_pool33", [2000, 1100], Hq=8, Hkv=2, w=8, pool="avg", pool_kernel=33, k=150, recipe="plant",
           plant_frac=0.02),
    W.Spec("r_pool33_max", [1537], Hq=8, Hkv=2, w=8, pool="max", pool_kernel=33, k=150, recipe="plant",
           plant_frac=0.02),
    W.Spec("r_R256", [1500, 700], Hq=32, Hkv=8, w=64, pool="avg", pool_kernel=7, k=120, recipe="plant"),
    W.Spec("r_R144", [1030], Hq=16, Hkv=2, w=18, pool="max", pool_kernel=5, k=60, recipe="plant"),
    W.Spec("r_many_blocks", [9000, 16, 40], Hq=16, Hkv=4, w=16, pool="max", pool_kernel=3,
           budgets=[[900, 1, 0, 9000], [16, 1, 0, 1], [40, 3, 39, 20]], recipe="plant", plant_frac=0.01),
]


@pytest.mark.parametrize("spec", EDGE, ids=lambda s: s.name)
def test_resident_edges_vs_oracle(kv, spec):
    _say(f"resident edge {spec.name} lens={spec.seq_lens} R={spec.rows * (spec.Hq // spec.Hkv)}")
    case = W.make_case(spec)
    out = _compress(kv, spec, case)
    ref = O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), **W.oracle_kwargs(spec))
    st = check_against_oracle(spec, case, out, ref)
    assert st["segments"] == spec.batch * spec.Hkv
    assert st["max_rel"] < 1e-4, st


FALLBACK = [W.small_cases()[i] for i in (2, 5, 7, 15, 19)] + [EDGE[3], EDGE[7]]


@pytest.mark.parametrize("spec", FALLBACK, ids=lambda s: s.name)
def test_late_blocks_give_the_same_bytes(kv, spec):
    """With no waiting at all, every block computes the statistics of the
    blocks that have not published yet: the same bytes come out."""
    _say(f"late-block path {spec.name}")
    case = W.make_case(spec)
    a = _compress(kv, spec, case)
    with _env(KVSEL_SPIN_CAP=0):
        b = _compress(kv, spec, case)
    for name in ("idx", "K_out", "V_out", "pooled"):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("spec", [W.small_cases()[i] for i in (3, 6, 7, 15, 20)], ids=lambda s: s.name)
def test_two_launch_scoring_still_matches(kv, spec):
    """kvsel_compress through the two-launch scoring: the oracle's result,
    and the resident path's up to fp32 rounding (pooled within 1e-5, kept
    sets equal up to near-ties)."""
    _say(f"two-launch compress {spec.name}")
    case = W.make_case(spec)
    res = _compress(kv, spec, case)
    with _env(KVSEL_FORCE_TWO_PASS=1):
        two = _compress(kv, spec, case)
    ref = O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), **W.oracle_kwargs(spec))
    check_against_oracle(spec, case, two, ref)
    pr = res["pooled"].cpu().numpy()
    pt = two["pooled"].cpu().numpy()
    ir = res["idx"].cpu().numpy()
    it = two["idx"].cpu().numpy()
    for (b, h, L, soff, ooff, keff) in segments(spec, res["out_offsets"]):
        check_scores(pr[soff:soff + L], pt[soff:soff + L], f"resident vs two-launch {(b, h)}", rtol=1e-5)
        check_selection(ir[ooff:ooff + keff], it[ooff:ooff + keff], pt[soff:soff + L].astype(np.float64), keff, L,
                        rtol=1e-5)


def test_c2_layer_all_heads_vs_two_launch(kv):
    """One Llama-shaped layer (L = 32768, 8 KV heads): the resident path's
    pooled scores against the two-launch path's on every head."""
    spec = W.config(2)
    _say("c2 layer: resident vs two-launch")
    case = W.make_case(spec, layer=5, device=DEV)
    res = _compress(kv, spec, case)
    with _env(KVSEL_FORCE_TWO_PASS=1):
        two = _compress(kv, spec, case)
    pr = res["pooled"].cpu().numpy()
    pt = two["pooled"].cpu().numpy()
    for (b, h, L, soff, ooff, keff) in segments(spec, res["out_offsets"]):
        check_scores(pr[soff:soff + L], pt[soff:soff + L], f"c2 {(b, h)}", rtol=1e-5)
