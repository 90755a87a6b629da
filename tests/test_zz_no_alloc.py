"""kvsel_compress_noalloc (the entry point that allocates nothing) on an
MI355X: through the C ABI, its outputs against kvsel_compress's on the same
inputs, byte for byte, for two calls in a row (the second on a smaller
problem, so the shared scratch holds the first call's bytes), and the clear
error for a problem whose workspace exceeds the scratch."""

import sys

import pytest
import torch

import workloads as W
from parity import Guarded

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def kv():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import attention_token_selection_amd as k

    return k


def _run_both(kv, spec):
    print(f"no-alloc vs workspace: {spec.name}", flush=True)
    sys.stdout.flush()
    case = W.make_case(spec)
    Q, K, V = (case[x].to(DEV) for x in "QKV")
    p = kv.Problem(**W.problem_kwargs(spec))
    ref = kv.compress(p, Q, K, V, pooled=True)
    g = Guarded(DEV)
    out = g.outputs(kv, p, pooled=True)
    kv.kvsel_compress_noalloc(p, Q, K, V, out["idx"], out["K_out"], out["V_out"], out["pooled"])
    g.check()
    kept = out["out_offsets"][-1]
    assert torch.equal(out["idx"][:kept], ref["idx"][:kept])
    assert torch.equal(out["K_out"][:kept], ref["K_out"][:kept])
    assert torch.equal(out["V_out"][:kept], ref["V_out"][:kept])
    assert torch.equal(out["pooled"], ref["pooled"])


def test_noalloc_matches_compress_twice_second_smaller(kv):
    big = W.config(1)  # one sequence of 4096 keys, 8 KV heads
    small = next(s for s in W.small_cases() if s.name == "s_ragged3")  # 3 sequences, 4 KV heads: fewer keys
    assert sum(small.seq_lens) * small.Hkv < sum(big.seq_lens) * big.Hkv
    _run_both(kv, big)
    _run_both(kv, small)


def test_noalloc_rejects_a_problem_past_its_scratch(kv):
    """The size check comes before anything is read or written: small dummy
    buffers stand in for the arguments, passed straight to the C function."""
    from attention_token_selection_amd.kvsel import KVSEL_EUNSUPPORTED, _lib

    p = kv.Problem(Hq=32, Hkv=8, w=32, L=1 << 20, k=4096, pool="max", pool_kernel=7)
    ws, _ = kv.kvsel_plan(p)
    assert ws > 64 << 20
    dummy = torch.zeros(4096, dtype=torch.uint8, device=DEV)
    ptr = dummy.data_ptr()
    with torch.cuda.device(DEV):
        st = _lib.kvsel_compress_noalloc(p.ref(), ptr, ptr, ptr, ptr, ptr, ptr, None, None)
    torch.cuda.synchronize()
    assert st == KVSEL_EUNSUPPORTED
    msg = _lib.kvsel_last_error().decode()
    assert "workspace" in msg and str(ws) in msg, msg
