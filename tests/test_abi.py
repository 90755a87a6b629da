"""The C ABI without a GPU: the library loads, exports what include/kvsel.h
declares, plans correctly and rejects bad arguments before touching a device."""

import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle.kvsel_oracle as O
import workloads as W

kv = pytest.importorskip("attention_token_selection_amd.kvsel")


def test_exports_every_declared_function():
    names = kv.exported_functions()
    assert set(names) >= {"kvsel_plan", "kvsel_score", "kvsel_row_stats", "kvsel_score_from_stats",
                          "kvsel_pool_topk", "kvsel_gather", "kvsel_compress", "kvsel_abi_version",
                          "kvsel_status_string", "kvsel_last_error"}
    lib = ctypes.CDLL(kv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    dyn = subprocess.run(["nm", "-D", "--defined-only", kv.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in dyn.splitlines() if " T " in line}
    assert set(names) <= exported
    # nothing else of ours leaks out of the library
    assert not [s for s in exported if s.startswith("_ZN5kvsel")]


def test_abi_version_matches_header():
    with open(kv.HEADER_PATH) as f:
        assert "#define KVSEL_ABI_VERSION 2" in f.read()
    assert kv.abi_version() == 2


def test_status_strings():
    for s in range(4):
        assert kv._lib.kvsel_status_string(s)
    assert kv._lib.kvsel_status_string(99) == b"unknown status"


@pytest.mark.parametrize("spec", W.small_cases() + [W.config(i) for i in range(1, 6)], ids=lambda s: s.name)
def test_plan_offsets_match_oracle(spec):
    p = kv.Problem(**W.problem_kwargs(spec))
    ws, offs = kv.kvsel_plan(p)
    budgets = spec.budgets or [[spec.k] * spec.Hkv for _ in spec.seq_lens]
    assert offs == O.plan_offsets(spec.seq_lens, spec.Hkv, budgets).tolist()
    # workspace holds at least the unpooled and pooled fp32 scores
    assert ws >= 2 * 4 * sum(spec.seq_lens) * spec.Hkv


def _status(p):
    ws = ctypes.c_size_t(0)
    return kv._lib.kvsel_plan(p.ref(), ctypes.byref(ws), None)


BAD = {
    "hq_not_multiple": dict(Hq=6, Hkv=4),
    "w_zero": dict(w=0),
    "w_too_long": dict(w=9),
    "even_pool": dict(pool="avg", pool_kernel=4),
    "zero_pool": dict(pool="max", pool_kernel=0),
    "alpha_big": dict(has_decode=True, alpha=1.5),
    "alpha_nan": dict(has_decode=True, alpha=float("nan")),
    "k_negative": dict(k=-1),
    "chunk_not_32": dict(key_chunk=48),
    "decode_flag": dict(has_decode=2),
    "scale_inf": dict(scale=float("inf")),
    "budget_negative": dict(budgets=[[1, -1]]),
    "weighting_unknown": dict(weighting=2),
    "lambda_negative": dict(weighting="exp", lam=-0.1),
    "lambda_nan": dict(weighting="exp", lam=float("nan")),
    "lambda_inf": dict(weighting="exp", lam=float("inf")),
    "sink_negative": dict(sink=-1),
    "recent_negative": dict(recent=-2),
    "gqa_unknown": dict(gqa=2),
    "stream_not_2048": dict(stream_keys=1000),
    "stream_negative": dict(stream_keys=-2048),
}


@pytest.mark.parametrize("name", sorted(BAD))
def test_plan_rejects_invalid(name):
    kw = dict(Hq=4, Hkv=2, w=2, L=8, k=2)
    kw.update(BAD[name])
    p = kv.Problem(**kw)
    if name == "decode_flag":
        p.struct.has_decode = 2
    assert _status(p) == kv.KVSEL_EINVAL, kv._lib.kvsel_last_error()
    assert kv._lib.kvsel_last_error()


def test_plan_rejects_bad_offsets_and_batch():
    p = kv.Problem(Hq=4, Hkv=2, w=2, seq_lens=[8, 0], k=1)
    assert _status(p) == kv.KVSEL_EINVAL
    p = kv.Problem(Hq=4, Hkv=2, w=2, L=8, k=1)
    p.struct.batch = 0
    assert _status(p) == kv.KVSEL_EINVAL
    assert kv._lib.kvsel_plan(None, ctypes.byref(ctypes.c_size_t()), None) == kv.KVSEL_EINVAL
    assert kv._lib.kvsel_plan(p.ref(), None, None) == kv.KVSEL_EINVAL


@pytest.mark.parametrize("kw", [dict(d=64), dict(Hq=65 * 2, Hkv=65), dict(Hq=32, Hkv=2, w=33),
                                dict(L=(1 << 20) + 1), dict(seq_lens=[100, (1 << 20) + 1], L=0)])
def test_plan_unsupported(kw):
    base = dict(Hq=4, Hkv=2, w=2, L=64, k=2)
    base.update(kw)
    assert _status(kv.Problem(**base)) == kv.KVSEL_EUNSUPPORTED


def test_longest_supported_sequence_plans():
    """2^20 keys is the longest sequence the selection supports."""
    assert _status(kv.Problem(Hq=4, Hkv=2, w=2, L=1 << 20, k=2)) == kv.KVSEL_OK


def test_key_chunk_caps_the_pass1_block():
    """key_chunk bounds the pass-1 block (TideKV's b_s): a chunk at or above
    the library's own block size changes nothing, and a smaller one means
    more blocks and so more per-block row records."""
    base = dict(Hq=32, Hkv=8, w=32, seq_lens=[4100, 2500], k=200)
    ws0 = kv.kvsel_plan(kv.Problem(**base))[0]
    assert kv.kvsel_plan(kv.Problem(**base, key_chunk=8192))[0] == ws0
    assert kv.kvsel_plan(kv.Problem(**base, key_chunk=512))[0] == ws0
    ws64 = kv.kvsel_plan(kv.Problem(**base, key_chunk=64))[0]
    ws32 = kv.kvsel_plan(kv.Problem(**base, key_chunk=32))[0]
    assert ws64 < ws32


def test_budget_clamping():
    p = kv.Problem(Hq=4, Hkv=2, w=1, seq_lens=[5, 3], budgets=[[0, 9], [3, 2]])
    _, offs = kv.kvsel_plan(p)
    assert offs == [0, 0, 5, 8, 10]


def _aligned_buffer(n):
    buf = (ctypes.c_char * (n + 512))()
    return buf, (ctypes.addressof(buf) + 255) // 256 * 256


def test_entry_points_validate_before_device():
    """Invalid pointers and sizes are caught on the host (EINVAL) even where no
    GPU exists; valid arguments then fail cleanly in the device check."""
    p = kv.Problem(Hq=4, Hkv=1, w=1, L=8, k=2)
    ws, _ = kv.kvsel_plan(p)
    buf, a = _aligned_buffer(ws)
    A = ctypes.c_void_p(a)
    lib = kv._lib
    sz = ctypes.c_size_t(ws)
    assert lib.kvsel_score(p.ref(), None, A, A, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_score(p.ref(), ctypes.c_void_p(a + 2), A, A, A, sz, None) == kv.KVSEL_EINVAL
    assert b"aligned" in lib.kvsel_last_error()
    assert lib.kvsel_score(p.ref(), A, A, A, A, ctypes.c_size_t(ws - 1), None) == kv.KVSEL_EINVAL
    assert b"too small" in lib.kvsel_last_error()
    assert lib.kvsel_score(p.ref(), A, A, A, ctypes.c_void_p(a + 16), sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_row_stats(p.ref(), A, None, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_row_stats(p.ref(), A, A, A, ctypes.c_size_t(ws - 1), None) == kv.KVSEL_EINVAL
    assert lib.kvsel_score_from_stats(p.ref(), A, A, None, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_pool_topk(p.ref(), A, None, None, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_gather(p.ref(), A, A, None, A, A, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_compress(p.ref(), A, A, A, A, A, None, None, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_profile_layer(p.ref(), A, A, None, 0, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_profile_layer(p.ref(), A, A, A, 2, A, sz, None) == kv.KVSEL_EINVAL
    assert b"accumulate" in lib.kvsel_last_error()
    assert lib.kvsel_profile_layer(p.ref(), A, A, A, 1, A, ctypes.c_size_t(ws - 1), None) == kv.KVSEL_EINVAL
    assert lib.kvsel_tier_rank(p.ref(), A, 1, 1, None, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_tier_rank(p.ref(), A, -1, 1, A, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_tier_rank(p.ref(), A, 1, -5, A, A, sz, None) == kv.KVSEL_EINVAL
    assert lib.kvsel_tier_rank(p.ref(), ctypes.c_void_p(a + 4), 1, 1, A, A, sz, None) == kv.KVSEL_EINVAL
    if not os.path.exists("/dev/kfd"):
        st = lib.kvsel_score(p.ref(), A, A, A, A, sz, None)
        assert st == kv.KVSEL_EHIP
        assert lib.kvsel_last_error()
    del buf


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    p = kv.Problem(Hq=4, Hkv=1, w=1, L=8, k=2)
    with pytest.raises(ValueError):
        kv.kvsel_score(p, torch.zeros(512, dtype=torch.bfloat16), torch.zeros(1024, dtype=torch.bfloat16),
                       torch.zeros(8), torch.zeros(10, dtype=torch.uint8))


def test_struct_layout_matches_c():
    """Offsets of kvsel_problem fields as a C compiler lays them out."""
    src = r'''
#include <stddef.h>
#include <stdio.h>
#include "kvsel.h"
#define F(x) printf("%s %zu\n", #x, offsetof(kvsel_problem, x));
int main(void) { F(batch) F(Hq) F(Hkv) F(d) F(L) F(seq_offsets_h) F(w) F(has_decode) F(alpha) F(causal)
  F(scale) F(pool) F(pool_kernel) F(k) F(budgets_h) F(key_chunk) F(weighting) F(lambda) F(sink_tokens)
  F(recent_tokens) F(gqa) F(stream_keys) printf("size %zu\n", sizeof(kvsel_problem)); return 0; }
'''
    import tempfile

    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        with open(c, "w") as f:
            f.write(src)
        subprocess.run(["gcc", "-I", os.path.dirname(kv.HEADER_PATH), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    got = dict(line.split() for line in out.splitlines())
    for name, _ in kv.KvselProblem._fields_:
        c_name = name.rstrip("_")  # "lambda" is a Python keyword
        assert int(got[c_name]) == getattr(kv.KvselProblem, name).offset, name
    assert int(got["size"]) == ctypes.sizeof(kv.KvselProblem)


# ---------------------------------------------------------------- host-only budget allocation
@pytest.mark.parametrize("seed", range(6))
def test_allocate_budgets_matches_oracle(seed):
    """The library's greedy (host C) makes the oracle's choices on random
    instances: concave top-k masses and arbitrary benefits, uneven sizes."""
    rng = np.random.default_rng(seed)
    sizes = [0, 64, 256, 512, 1024, 4096] if seed % 2 else [16, 17, 40, 41, 300]
    items = int(rng.integers(1, 70))
    if seed < 3:
        benefit = np.stack([O.topk_mass(rng.random(4096) ** 4, sizes) for _ in range(items)])
    else:
        benefit = rng.random((items, len(sizes))) * 10
    for total in (0, sizes[0] * items, sizes[0] * items + 1, 500 * items, 10 ** 9):
        got = kv.kvsel_allocate_budgets(benefit, sizes, total)
        want = np.asarray(sizes)[O.greedy_allocate(benefit, sizes, total)]
        np.testing.assert_array_equal(got, want)
        if total >= sizes[0] * items:
            assert int(got.astype(np.int64).sum()) <= total


def test_allocate_budgets_hand_and_validation():
    assert kv.kvsel_allocate_budgets([[0, 5, 6], [0, 3, 6], [0, 1, 11]], [0, 2, 4], 6).tolist() == [2, 4, 0]
    assert kv.kvsel_allocate_budgets(np.zeros((0, 2)), [0, 1], 5).tolist() == []
    for bad in (([[0, 1]], [1, 1], 5), ([[0, 1]], [-1, 1], 5), ([[0, float("nan")]], [0, 1], 5)):
        with pytest.raises(kv.KvselError):
            kv.kvsel_allocate_budgets(*bad)


def test_streaming_workspace_is_bounded():
    """With stream_keys the workspace does not grow with the prefix length."""
    whole = kv.kvsel_plan(kv.Problem(Hq=32, Hkv=8, w=32, L=1 << 20, pool="max", pool_kernel=7, k=2048))[0]
    # 16384 and 32768 keys per step: the step-wise form (the running row of
    # the budget plus a step exceeds the fused selection's); 8192: the fused form
    for C in (32768, 8192, 16384):
        sizes = []
        for L in (4000, 4096, 65536, 1 << 20):
            p = kv.Problem(Hq=32, Hkv=8, w=32, L=L, pool="max", pool_kernel=7, k=2048, stream_keys=C)
            sizes.append(kv.kvsel_plan(p)[0])
        assert len(set(sizes)) == 1, (C, sizes)
        assert sizes[0] * 8 < whole
    # budgets too large for one candidate row
    p = kv.Problem(Hq=4, Hkv=1, w=1, L=1 << 20, k=1 << 20, stream_keys=2048)
    assert _status(p) == kv.KVSEL_EUNSUPPORTED


def test_streaming_rejected_by_whole_prefix_entry_points():
    p = kv.Problem(Hq=4, Hkv=1, w=1, L=8, k=2, stream_keys=2048)
    ws, _ = kv.kvsel_plan(p)
    buf, a = _aligned_buffer(ws)
    A = ctypes.c_void_p(a)
    lib = kv._lib
    sz = ctypes.c_size_t(ws)
    for st in (lib.kvsel_score(p.ref(), A, A, A, A, sz, None), lib.kvsel_row_stats(p.ref(), A, A, A, sz, None),
               lib.kvsel_pool_topk(p.ref(), A, A, A, A, sz, None),
               lib.kvsel_compress(p.ref(), A, A, A, A, A, A, A, A, sz, None)):
        assert st == kv.KVSEL_EINVAL
    del buf
