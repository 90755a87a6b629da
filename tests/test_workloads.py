"""The seeded input generator: deterministic, right shapes, right structure."""

import math

import torch

import workloads as W


def test_deterministic_and_bf16():
    spec = W.small_cases()[6]
    a = W.make_case(spec, layer=0)
    b = W.make_case(spec, layer=0)
    c = W.make_case(spec, layer=1)
    for key in "QKV":
        assert a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])


def test_shapes_of_every_config():
    for i in range(1, 6):
        s = W.config(i)
        assert s.Hq == 32 and s.Hkv == 8 and s.d == 128
        assert len(s.seq_lens) == s.batch
    assert W.config(2).layers == 32 and W.config(2).seq_lens == [32768]
    assert W.config(3).key_chunk == 4096 and W.config(3).w == 64
    s5 = W.config(5)
    assert all(8192 <= L <= 65536 for L in s5.seq_lens)
    assert all(256 <= k <= 4096 for row in s5.budgets for k in row)


def test_small_case_shapes_and_plants():
    spec = W.config(1)
    case = W.make_case(spec)
    assert case["Q"].shape == (1, 32, 32, 128)
    assert case["K"].shape == (4096, 8, 128)
    K = case["K"].float()
    # planted keys are longer along their head's direction: roughly 82 positions
    # stand out in norm (|k|^2 ~ 1 + 2.25)
    n2 = (K ** 2).sum(-1)[:, 0]
    assert 60 <= int((n2 > 2.4).sum()) <= 110
    q = case["Q"].float()[0, :, 0, :]
    assert 0.7 * math.sqrt(128) < q.std().item() < 1.5 * math.sqrt(128)


def test_run_positions_are_clustered():
    g = torch.Generator().manual_seed(3)
    pos = W._run_positions(g, 32768, 328)
    assert len(pos) == 328
    gaps = (pos[1:] - pos[:-1])
    assert (gaps == 1).sum() > 100  # most positions sit inside runs


def test_decode_correlation():
    spec = W.small_cases()[5]
    case = W.make_case(spec)
    qd = case["Q"].float()[0, spec.w, 0, :]
    K = case["K"].float()[:, 0, :]
    cos = (K @ qd) / (K.norm(dim=1) * qd.norm())
    assert int((cos > 0.65).sum()) >= 1
    assert torch.isclose(cos.max(), torch.tensor(0.7), atol=0.02)
