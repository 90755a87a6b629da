"""Seeded synthetic inputs for attention-score-based KV-cache selection.

This module only draws inputs.  It holds none of the selection arithmetic
(no softmax, pooling, top-k or gather), so the fp64 oracle and the HIP path
can both consume its output without sharing any of the method's code.

Geometry is Llama-3.1-8B-like (32 query heads, 8 KV heads, head dim 128), as
on the TideKV page (§6.1, evaluation setup).  No dataset is available, so
seeded random tensors with the structure below stand in for the long-context
benchmark prompts the pages evaluate on (LongBench / RULER lengths 4K-128K,
budgets 256-4096, observation windows of 16-64 rows).

Conventions shared by every workload:

* Values are drawn in fp32 from a ``torch.Generator`` seeded per
  (workload, layer, stream) and rounded once to bf16 (round to nearest even).
* Keys and values: i.i.d. N(0, 1)/sqrt(d).
* Window queries: i.i.d. N(0, d) per component, so background logits
  ``q.k/sqrt(d)`` are about N(0, 1).
* Planted positions: key += 1.5 * u_h and the group's window queries
  += 2*sqrt(d) * u_h for a unit direction u_h per KV head, which adds about
  3 to the logit of a planted key.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import List, Optional

import torch

BASE_SEED = 20261202


@dataclasses.dataclass
class Spec:
    """A workload: shapes, selection parameters and the input recipe."""

    name: str
    seq_lens: List[int]
    Hq: int = 32
    Hkv: int = 8
    d: int = 128
    w: int = 32
    has_decode: bool = False
    alpha: float = 0.0
    causal: bool = True
    scale: float = 0.0  # 0 -> 1/sqrt(d)
    pool: str = "none"  # none | avg | max
    pool_kernel: int = 1
    k: int = 0
    budgets: Optional[List[List[int]]] = None  # [B][Hkv]
    key_chunk: int = 0
    weighting: str = "alpha"  # alpha | exp (temporal row weights)
    lam: float = 0.0  # exp weighting: c_r proportional to exp(lam * r)
    sink: int = 0  # reserved prefix positions
    recent: int = 0  # reserved suffix positions
    gqa: str = "sum"  # sum (per-head softmax, summed) | mean (one mean query per group)
    layers: int = 1
    recipe: str = "plant"  # plant | runs | zipf | decode_corr | plain | hand
    plant_frac: float = 0.02
    seed_tag: int = 0

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def rows(self) -> int:
        return self.w + (1 if self.has_decode else 0)

    def budget(self, b: int, h: int) -> int:
        return self.budgets[b][h] if self.budgets is not None else self.k


def _seed(*parts) -> int:
    h = hashlib.sha256(repr((BASE_SEED,) + parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _unit(g, n, d, device):
    u = torch.randn(n, d, generator=g, device=device, dtype=torch.float32)
    return u / u.norm(dim=1, keepdim=True)


def _isolated_positions(g, L, count, device):
    perm = torch.randperm(L, generator=g, device=device)
    return perm[:count].sort().values


def _run_positions(g, L, count):
    """Positions in non-overlapping runs of 1..16 tokens (last run truncated)."""
    taken = torch.zeros(L, dtype=torch.bool)
    total = 0
    while total < count:
        run = int(torch.randint(1, 17, (1,), generator=g).item())
        run = min(run, count - total)
        start = int(torch.randint(0, L - run + 1, (1,), generator=g).item())
        if taken[max(0, start - 1):start + run + 1].any():
            continue  # keep runs separate
        taken[start:start + run] = True
        total += run
    return taken.nonzero().flatten()


def make_case(spec: Spec, layer: int = 0, device="cpu"):
    """Draw Q [B, w', Hq, d], K and V [sum L_b, Hkv, d] (bf16) for one layer."""
    dev = torch.device(device)
    gdev = "cuda" if dev.type == "cuda" else "cpu"
    d, Hq, Hkv = spec.d, spec.Hq, spec.Hkv
    G = Hq // Hkv
    Ks, Vs, Qs = [], [], []
    for b, L in enumerate(spec.seq_lens):
        g = _gen(gdev, spec.name, spec.seed_tag, layer, b)
        K = torch.randn(L, Hkv, d, generator=g, device=dev) / math.sqrt(d)
        V = torch.randn(L, Hkv, d, generator=g, device=dev) / math.sqrt(d)
        Q = torch.randn(spec.rows, Hq, d, generator=g, device=dev) * math.sqrt(d)
        if spec.recipe in ("plant", "runs"):
            n = max(1, round(spec.plant_frac * L))
            if spec.recipe == "plant":
                pos = _isolated_positions(g, L, n, gdev).to(dev)
            else:
                pos = _run_positions(torch.Generator().manual_seed(_seed(spec.name, layer, b, "runs")), L, n).to(dev)
            u = _unit(g, Hkv, d, dev)  # one direction per KV head
            K[pos] += 1.5 * u[None, :, :]
            gamma = 2.0 * math.sqrt(d)
            Q[: spec.w] += gamma * u.repeat_interleave(G, dim=0)[None, :, :]
        elif spec.recipe == "zipf":
            uu = torch.rand(L, generator=g, device=dev)
            K *= (1.0 + 2.0 * uu.pow(8))[:, None, None]
        elif spec.recipe == "decode_corr":
            n = max(1, round(0.005 * L))
            pos = _isolated_positions(g, L, n, gdev).to(dev)
            v = _unit(g, Hkv, d, dev)
            ks = K[pos]  # [n, Hkv, d]
            norm = ks.norm(dim=2, keepdim=True)
            along = (ks * v[None]).sum(dim=2, keepdim=True)
            perp = ks - along * v[None]
            perp = perp / perp.norm(dim=2, keepdim=True)
            K[pos] = norm * (0.7 * v[None] + math.sqrt(1.0 - 0.49) * perp)
            if spec.has_decode:
                Q[spec.w] = d * v.repeat_interleave(G, dim=0)
        elif spec.recipe == "plain":
            pass
        else:
            raise ValueError(spec.recipe)
        Ks.append(K)
        Vs.append(V)
        Qs.append(Q)
    return {
        "Q": torch.stack(Qs).to(torch.bfloat16).contiguous(),
        "K": torch.cat(Ks).to(torch.bfloat16).contiguous(),
        "V": torch.cat(Vs).to(torch.bfloat16).contiguous(),
    }


def hand_case(keys_c0, q_c0, Hq, Hkv, d=128):
    """Tiny exact inputs: only component 0 is nonzero (one sequence).

    ``keys_c0`` [L] applies to every KV head; ``q_c0`` [w'][Hq].
    """
    L = len(keys_c0)
    K = torch.zeros(L, Hkv, d)
    K[:, :, 0] = torch.tensor(keys_c0, dtype=torch.float32)[:, None]
    V = torch.zeros(L, Hkv, d)
    V[:, :, 0] = torch.arange(L, dtype=torch.float32)[:, None]
    V[:, :, 1] = torch.arange(Hkv, dtype=torch.float32)[None, :]
    Q = torch.zeros(1, len(q_c0), Hq, d)
    Q[0, :, :, 0] = torch.tensor(q_c0, dtype=torch.float32)
    return {"Q": Q.to(torch.bfloat16), "K": K.to(torch.bfloat16), "V": V.to(torch.bfloat16)}


def _budgets(tag, B, Hkv, lo, hi):
    g = torch.Generator().manual_seed(_seed("budgets", tag))
    return torch.randint(lo, hi + 1, (B, Hkv), generator=g).tolist()


def _lengths(tag, B, lo, hi):
    g = torch.Generator().manual_seed(_seed("lengths", tag))
    return torch.randint(lo, hi + 1, (B,), generator=g).tolist()


def config(i: int) -> Spec:
    """The five reference workloads (1-based numbering as listed)."""
    if i == 1:
        return Spec("c1_L4k_avg7_k512", [4096], w=32, pool="avg", pool_kernel=7, k=512,
                    recipe="plant", plant_frac=0.02)
    if i == 2:
        return Spec("c2_32layers_L32k_max7_k2048", [32768], w=32, pool="max", pool_kernel=7, k=2048,
                    recipe="runs", plant_frac=0.01, layers=32)
    if i == 3:
        return Spec("c3_L128k_w64_chunk4096_avg7_k4096", [131072], w=64, pool="avg", pool_kernel=7,
                    k=4096, key_chunk=4096, recipe="zipf")
    if i == 4:
        return Spec("c4_B4_L64k_decode_a05_max5_k2048", [65536] * 4, w=32, has_decode=True, alpha=0.5,
                    pool="max", pool_kernel=5, k=2048, recipe="decode_corr")
    if i == 5:
        B = 8
        return Spec("c5_ragged8_avg7_headbudgets", _lengths("c5", B, 8192, 65536), w=32, pool="avg",
                    pool_kernel=7, budgets=_budgets("c5", B, 8, 256, 4096), recipe="plant",
                    plant_frac=0.01)
    raise ValueError(i)


def deferkv_full() -> Spec:
    """The DeferKV guide's defaults (lambda 0.1, 16 sinks, 32 recent) on the
    32K-key Llama-3.1-8B-like layer, with the decode-step row."""
    return Spec("deferkv_L32k_exp0.1_sink16_recent32_max7_k2048", [32768], w=32, has_decode=True, pool="max",
                pool_kernel=7, k=2048, weighting="exp", lam=0.1, sink=16, recent=32, recipe="decode_corr")


def deferkv_guide_full() -> Spec:
    """The guide's whole recipe on the same layer: its defaults plus the
    group's queries averaged into one query per row."""
    return dataclasses.replace(deferkv_full(), name="deferkv_L32k_meanq_exp0.1_sink16_recent32_max7_k2048",
                               gqa="mean")


def small_cases():
    """Small shapes spanning several key tiles, ragged tails and edge cases."""
    cases = [
        Spec("s_L1_w1", [1], Hq=4, Hkv=1, w=1, k=1, recipe="plain"),
        Spec("s_L5_k0", [5], Hq=4, Hkv=2, w=3, k=0, recipe="plain"),
        Spec("s_L17_kbig", [17], Hq=8, Hkv=2, w=5, pool="max", pool_kernel=3, k=100, recipe="plant",
             plant_frac=0.1),
        Spec("s_L33_avg5", [33], Hq=8, Hkv=8, w=33, pool="avg", pool_kernel=5, k=7, recipe="plain"),
        Spec("s_L100_nocausal", [100], Hq=32, Hkv=8, w=8, causal=False, pool="avg", pool_kernel=7, k=20,
             recipe="plant", plant_frac=0.05),
        Spec("s_L257_decode", [257], Hq=32, Hkv=8, w=16, has_decode=True, alpha=0.3, pool="max",
             pool_kernel=5, k=31, recipe="decode_corr"),
        Spec("s_L1000_w64", [1000], Hq=32, Hkv=8, w=64, pool="avg", pool_kernel=7, k=64, recipe="plant",
             plant_frac=0.02),
        Spec("s_ragged3", [300, 77, 1031], Hq=16, Hkv=4, w=12, pool="max", pool_kernel=7,
             budgets=[[5, 300, 0, 64], [77, 1, 80, 13], [100, 257, 1031, 2000]], recipe="plant",
             plant_frac=0.03),
        Spec("s_G1_scale", [513], Hq=8, Hkv=8, w=4, scale=0.05, pool="none", k=40, recipe="plant"),
        Spec("s_alpha1", [400], Hq=8, Hkv=2, w=8, has_decode=True, alpha=1.0, pool="avg", pool_kernel=3,
             k=50, recipe="decode_corr"),
        Spec("s_alpha0", [400], Hq=8, Hkv=2, w=8, has_decode=True, alpha=0.0, pool="avg", pool_kernel=3,
             k=50, recipe="decode_corr"),
        Spec("s_chunked", [4100], Hq=32, Hkv=8, w=32, pool="avg", pool_kernel=7, k=300, key_chunk=512,
             recipe="zipf"),
        Spec("s_w_big", [300], Hq=32, Hkv=8, w=128, pool="max", pool_kernel=7, k=33, recipe="plant"),
        Spec("s_many_seqs", [40 + 13 * i for i in range(10)], Hq=16, Hkv=8, w=4, pool="avg", pool_kernel=3,
             k=9, recipe="plant", plant_frac=0.05),
        Spec("s_hkv64", [70], Hq=64, Hkv=64, w=3, pool="max", pool_kernel=3, k=10, recipe="plain"),
        # DeferKV-style: exponential temporal row weights and reserved sink / recent positions
        Spec("s_exp_sink_recent", [3000], Hq=32, Hkv=8, w=32, has_decode=True, pool="max", pool_kernel=7,
             k=200, weighting="exp", lam=0.1, sink=16, recent=32, recipe="decode_corr"),
        Spec("s_exp_nodecode", [700], Hq=16, Hkv=4, w=16, pool="avg", pool_kernel=5, k=60, weighting="exp",
             lam=0.5, recipe="plant", plant_frac=0.05),
        Spec("s_reserve_over_budget", [500, 90], Hq=8, Hkv=2, w=8, pool="avg", pool_kernel=3,
             budgets=[[10, 40], [90, 3]], sink=8, recent=24, recipe="plant"),
        Spec("s_reserve_whole_seq", [2100], Hq=8, Hkv=2, w=8, has_decode=True, weighting="exp", lam=2.0,
             pool="max", pool_kernel=3, k=2090, sink=2100, recent=0, recipe="plain"),
        # the guide's mean-query grouped attention
        Spec("s_meanq_guide", [2500, 700], Hq=32, Hkv=8, w=32, has_decode=True, pool="max", pool_kernel=7, k=150,
             weighting="exp", lam=0.1, sink=16, recent=32, gqa="mean", recipe="decode_corr"),
        Spec("s_meanq_G3_alpha", [1000], Hq=12, Hkv=4, w=20, has_decode=True, alpha=0.5, pool="avg",
             pool_kernel=5, k=90, gqa="mean", recipe="plant", plant_frac=0.03),
        Spec("s_meanq_G1", [333], Hq=4, Hkv=4, w=5, pool="none", k=40, gqa="mean", recipe="plant"),
        # 4 n + 1 row tiles per KV head: n whole tiles per wave, the last one split into four 16 x 16
        # blocks (one per wave); five tiles (129 to 160 rows), nine (257 to 288), thirteen (385 to 416)
        Spec("s_R160_split5", [517, 4100], Hq=32, Hkv=8, w=39, has_decode=True, alpha=0.2, pool="avg",
             pool_kernel=3, k=100, recipe="plant"),
        Spec("s_R130_G2_nocausal", [2049, 64], Hq=16, Hkv=8, w=64, has_decode=True, alpha=0.7, causal=False,
             pool="max", pool_kernel=5, k=77, recipe="decode_corr"),
        Spec("s_R260_split9", [700, 1500], Hq=32, Hkv=8, w=64, has_decode=True, alpha=0.5, pool="max",
             pool_kernel=5, k=100, recipe="decode_corr"),
        Spec("s_R388_split13", [900], Hq=16, Hkv=4, w=96, has_decode=True, alpha=0.4, pool="avg",
             pool_kernel=3, k=150, recipe="plant"),
        # one KV head, G = 8: 8 x 18 = 144 rows, five row tiles
        Spec("s_R144_G8_split5", [1500, 333], Hq=8, Hkv=1, w=17, has_decode=True, alpha=0.6, pool="max",
             pool_kernel=3, k=120, recipe="decode_corr"),
        # a caller's key_chunk below the library's own block size: the cap binds (64-key blocks)
        Spec("s_chunk64_binds", [4100, 2500], Hq=32, Hkv=8, w=32, pool="avg", pool_kernel=5, k=200,
             key_chunk=64, recipe="zipf"),
    ]
    return cases


def problem_kwargs(spec: Spec) -> dict:
    """Keyword arguments describing ``spec`` to the library binding's Problem."""
    return dict(Hq=spec.Hq, Hkv=spec.Hkv, d=spec.d, w=spec.w, seq_lens=list(spec.seq_lens),
                has_decode=spec.has_decode, alpha=spec.alpha, causal=spec.causal, scale=spec.scale,
                pool=spec.pool, pool_kernel=spec.pool_kernel, k=spec.k, budgets=spec.budgets,
                key_chunk=spec.key_chunk, weighting=spec.weighting, lam=spec.lam, sink=spec.sink,
                recent=spec.recent, gqa=spec.gqa)


def oracle_kwargs(spec: Spec) -> dict:
    """Keyword arguments describing ``spec`` to the oracle's ``compress``."""
    return dict(seq_lens=list(spec.seq_lens), Hq=spec.Hq, Hkv=spec.Hkv, w=spec.w, has_decode=spec.has_decode,
                alpha=spec.alpha, causal=spec.causal, scale=(spec.scale if spec.scale else None), pool=spec.pool,
                pool_kernel=spec.pool_kernel, k=spec.k, budgets=spec.budgets, weighting=spec.weighting,
                lam=spec.lam, sink=spec.sink, recent=spec.recent, gqa=spec.gqa)
