"""kvsel_compress with the pool and the selection tables fused into pass 2,
on an MI355X.

kvsel_compress takes this path for pools up to 33 wide: pass 2 also scores
16 keys past each end of its block, pools, writes the pooled scores and
counting-sorts each 256 positions by a first digit; the selection launch
reads those tables.  These tests pin what is particular to it:

* shapes at the path's edges against the oracle: one key, table blocks of
  exactly 256 and 512 keys and one key more, a 33-wide pool (the halo's
  full 16 keys), a split row tile (R = 144), 256 rows, many blocks, budgets,
  reserved positions, a decode row, exponential weights;
* the same bytes as the unfused path (pass 2 writes S, then the separate
  pool and selection launches; KVSEL_UNFUSED=1): pooled scores, kept
  indices and the gathered rows;
* a 35-wide pool (past the halo) takes the unfused path and still matches
  the oracle.
"""

import os
import sys

import numpy as np
import pytest
import torch

import oracle.kvsel_oracle as O
import workloads as W
from parity import check_against_oracle, compress_guarded, to_np64

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
    out = compress_guarded(kv, p, *(case[x].to(DEV) for x in "QKV"), pooled=True)
    torch.cuda.synchronize()
    return out


EDGE = [
    W.Spec("f_L1", [1], Hq=4, Hkv=1, w=1, pool="avg", pool_kernel=5, k=1, recipe="plain"),
    W.Spec("f_L256", [256], Hq=32, Hkv=8, w=32, pool="max", pool_kernel=7, k=100, recipe="plant"),
    W.Spec("f_L257", [257], Hq=32, Hkv=8, w=32, pool="avg", pool_kernel=7, k=100, recipe="plant"),
    W.Spec("f_L512", [512], Hq=32, Hkv=8, w=32, pool="max", pool_kernel=7, k=100, recipe="plant"),
    W.Spec("f_L513", [513], Hq=32, Hkv=8, w=32, pool="avg", pool_kernel=7, k=100, recipe="plant"),
    W.Spec("f_pool33", [2000, 1100], Hq=8, Hkv=2, w=8, pool="avg", pool_kernel=33, k=150, recipe="plant",
           plant_frac=0.02),
    W.Spec("f_pool33_max", [1537], Hq=8, Hkv=2, w=8, pool="max", pool_kernel=33, k=150, recipe="plant",
           plant_frac=0.02),
    W.Spec("f_nopool", [3000], Hq=8, Hkv=2, w=8, pool="none", k=300, recipe="plant"),
    W.Spec("f_R256", [1500, 700], Hq=32, Hkv=8, w=64, pool="avg", pool_kernel=7, k=120, recipe="plant"),
    W.Spec("f_R144_split", [1030], Hq=16, Hkv=2, w=18, pool="max", pool_kernel=5, k=60, recipe="plant"),
    W.Spec("f_many_blocks", [9000, 16, 40], Hq=16, Hkv=4, w=16, pool="max", pool_kernel=3,
           budgets=[[900, 1, 0, 9000], [16, 1, 0, 1], [40, 3, 39, 20]], recipe="plant", plant_frac=0.01),
    W.Spec("f_decode_sink", [3100], Hq=8, Hkv=2, w=8, has_decode=True, alpha=0.3, pool="avg", pool_kernel=9,
           k=400, sink=4, recent=16, recipe="plant"),
    W.Spec("f_expw", [2600, 900], Hq=8, Hkv=2, w=8, weighting="exp", lam=0.2, pool="max", pool_kernel=5, k=250,
           recipe="plant"),
    W.Spec("f_pool35_unfused", [2000], Hq=8, Hkv=2, w=8, pool="avg", pool_kernel=35, k=150, recipe="plant"),
    # every score equal (logits scaled to nothing, no mask), so every key lands in the
    # threshold's bin: 3000 candidates (held in LDS, past direct ranking) and 9000 (past
    # the LDS, read from the buckets); ties go to the lower position
    W.Spec("f_ties_lds", [3000], Hq=8, Hkv=2, w=8, causal=False, scale=1e-30, pool="max", pool_kernel=3, k=500,
           recipe="plain"),
    W.Spec("f_ties_mem", [9000], Hq=8, Hkv=2, w=8, causal=False, scale=1e-30, pool="avg", pool_kernel=5, k=700,
           recipe="plain"),
]


@pytest.mark.parametrize("spec", EDGE, ids=lambda s: s.name)
def test_fused_edges_vs_oracle(kv, spec):
    _say(f"fused edge {spec.name} lens={spec.seq_lens} R={spec.rows * (spec.Hq // spec.Hkv)}")
    case = W.make_case(spec)
    out = _compress(kv, spec, case)
    ref = O.compress(to_np64(case["Q"]), to_np64(case["K"]), to_np64(case["V"]), **W.oracle_kwargs(spec))
    st = check_against_oracle(spec, case, out, ref)
    assert st["segments"] == spec.batch * spec.Hkv
    assert st["max_rel"] < 1e-4, st


SAME = [W.small_cases()[i] for i in (2, 3, 5, 6, 7, 15, 19, 20)] + [EDGE[i] for i in (0, 2, 5, 9, 10, 11, 14, 15)]


@pytest.mark.parametrize("spec", SAME, ids=lambda s: s.name)
def test_fused_and_unfused_give_the_same_bytes(kv, spec):
    """Pass 2 computes every key's S by the same steps in either form, the
    halo keys' included, and the pool sums in the same order: the pooled
    scores, the kept indices and the gathered rows agree byte for byte."""
    _say(f"fused vs unfused {spec.name}")
    case = W.make_case(spec)
    a = _compress(kv, spec, case)
    with _env(KVSEL_UNFUSED=1):
        b = _compress(kv, spec, case)
    for name in ("pooled", "idx", "K_out", "V_out"):
        assert torch.equal(a[name], b[name]), name


def test_c2_layer_fused_and_unfused_agree(kv):
    """One Llama-shaped layer (L = 32768, 8 KV heads), every head: the same
    bytes from both forms."""
    spec = W.config(2)
    _say("c2 layer: fused vs unfused")
    case = W.make_case(spec, layer=5, device=DEV)
    a = _compress(kv, spec, case)
    with _env(KVSEL_UNFUSED=1):
        b = _compress(kv, spec, case)
    for name in ("pooled", "idx", "K_out", "V_out"):
        assert torch.equal(a[name], b[name]), name
