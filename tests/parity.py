"""Comparison of the HIP path's outputs with the fp64 oracle.

Tolerances (fp32 accumulation of exact bf16 products, fp32 exp2; fp64 oracle):
* pooled and unpooled scores: |gpu - ref| <= RTOL * max(ref, 1e-12 * sum(ref))
  per position, RTOL = 2e-3 (the floor only keeps fp32 underflow of negligible
  entries from failing);
* kept positions: same count, ascending, and any position in one set but not
  the other must have an oracle pooled score within RTOL of the oracle's k-th
  largest value (several selections are correct near ties); reserved (sink and
  recent) positions are kept first, so the k-th value is taken over the others
  with the budget left after them;
* gathered K/V: bit-exact copies of the rows the GPU chose.
A second, tighter band (DIAG_RTOL) is reported, not enforced.

Every output buffer and workspace the GPU tests hand to the library sits
between two guard bands of a known byte pattern (``Guarded``); the bands are
checked after the calls, so a write past either end of a buffer fails.
"""

from __future__ import annotations

import numpy as np

RTOL = 2e-3
DIAG_RTOL = 1e-5


class Guarded:
    """Device buffers with GUARD bytes of a fixed pattern on each side.

    ``empty(n, dtype)`` returns an n-element view (256-byte aligned) inside a
    larger allocation; ``check()`` asserts that no guard byte changed."""

    GUARD = 4096

    def __init__(self, device):
        import torch

        self.device = device
        self.bufs = []
        self.pattern = (torch.arange(self.GUARD, dtype=torch.int32, device=device) * 37 % 251 + 3).to(torch.uint8)

    def empty(self, n, dtype, fill=None):
        import torch

        elt = torch.empty((), dtype=dtype).element_size()
        nbytes = (n * elt + 255) // 256 * 256
        raw = torch.empty(self.GUARD + nbytes + self.GUARD, dtype=torch.uint8, device=self.device)
        raw[:self.GUARD] = self.pattern
        raw[self.GUARD + nbytes:] = self.pattern
        view = raw[self.GUARD:self.GUARD + n * elt].view(dtype)
        if fill is not None:
            view.fill_(fill)
        self.bufs.append((raw, nbytes))
        return view

    def outputs(self, kv, problem, pooled=True):
        """Like kvsel.alloc_outputs, every buffer guarded."""
        import torch

        ws, offs = kv.kvsel_plan(problem)
        kept = offs[-1]
        n = sum(problem.seq_lens) * problem.Hkv
        return {
            "idx": self.empty(max(kept, 1), torch.int32),
            "K_out": self.empty(max(kept, 1) * problem.d, torch.bfloat16).view(max(kept, 1), problem.d),
            "V_out": self.empty(max(kept, 1) * problem.d, torch.bfloat16).view(max(kept, 1), problem.d),
            "pooled": self.empty(max(n, 1), torch.float32) if pooled else None,
            "ws": self.empty(ws, torch.uint8),
            "out_offsets": offs,
        }

    def check(self):
        import torch

        torch.cuda.synchronize()
        for i, (raw, nbytes) in enumerate(self.bufs):
            head = raw[:self.GUARD]
            tail = raw[self.GUARD + nbytes:]
            assert torch.equal(head, self.pattern), f"guarded buffer {i}: bytes before it were written"
            assert torch.equal(tail, self.pattern), f"guarded buffer {i}: bytes past its end were written"


def compress_guarded(kv, problem, Q, K, V, pooled=True):
    """kvsel_compress on guarded outputs and workspace; checks the guards."""
    g = Guarded(K.device)
    out = g.outputs(kv, problem, pooled=pooled)
    kv.kvsel_compress(problem, Q, K, V, out["idx"], out["K_out"], out["V_out"], out["pooled"], out["ws"])
    g.check()
    out["guard"] = g
    return out


def to_np64(t):
    import torch

    return t.detach().to("cpu", torch.float64).numpy()


def check_scores(gpu, ref, what="scores", rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = 1e-12 * ref.sum()
    bound = rtol * np.maximum(ref, floor)
    err = np.abs(gpu - ref)
    bad = np.nonzero(err > bound)[0]
    if len(bad):
        i = bad[0]
        raise AssertionError(f"{what}: {len(bad)} positions beyond {rtol:g} relative; first at {i}: "
                             f"gpu={gpu[i]!r} ref={ref[i]!r}")
    denom = np.maximum(ref, floor)
    # an all-zero reference segment has no scale: exact zeros count as 0 error
    rel = np.where(denom > 0, err / np.where(denom > 0, denom, 1.0), np.where(err > 0, np.inf, 0.0))
    return {"max_rel": float(rel.max()) if len(rel) else 0.0,
            "beyond_diag": int((rel > DIAG_RTOL).sum())}


def kth_value(P, k):
    if k <= 0:
        return np.inf
    order = np.lexsort((np.arange(len(P)), -P))
    return P[order[k - 1]]


def reserved_mask(L, sink=0, recent=0):
    """Positions always kept: the first ``sink`` and the last ``recent``."""
    m = np.zeros(L, dtype=bool)
    m[:min(sink, L)] = True
    if recent > 0:
        m[max(0, L - recent):] = True
    return m


def check_selection(gpu_idx, ref_idx, P_ref, keff, L, rtol=RTOL, reserved=None):
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    ref_idx = np.asarray(ref_idx, dtype=np.int64)
    assert len(gpu_idx) == keff == len(ref_idx), (len(gpu_idx), keff, len(ref_idx))
    if keff == 0:
        return 0
    assert np.all(np.diff(gpu_idx) > 0), "positions must be strictly ascending"
    assert gpu_idx[0] >= 0 and gpu_idx[-1] < L
    diff = np.setxor1d(gpu_idx, ref_idx)
    if reserved is not None and reserved.any():
        # reserved positions are not chosen by score: both sides keep the same ones
        assert not reserved[diff].any(), f"reserved positions {diff[reserved[diff]][:10]} differ"
        others = np.nonzero(~reserved)[0]
        tau = kth_value(P_ref[others], keff - int(reserved.sum()))
    else:
        tau = kth_value(P_ref, keff)
    near = np.abs(P_ref[diff] - tau) <= rtol * tau
    assert np.all(near), f"positions {diff[~near][:10]} differ and are not near-ties (tau={tau})"
    return len(diff)


def _runs(mask, limit=6):
    """(first, last) index of the first few runs of True in a boolean array."""
    idx = np.nonzero(mask)[0]
    if not len(idx):
        return []
    br = np.nonzero(np.diff(idx) > 1)[0]
    starts = np.concatenate([[idx[0]], idx[br + 1]])
    ends = np.concatenate([idx[br], [idx[-1]]])
    return list(zip(starts.tolist(), ends.tolist()))[:limit]


def check_finite(x, what):
    x = np.asarray(x)
    bad = ~np.isfinite(x)
    assert not bad.any(), f"{what}: {int(bad.sum())} non-finite values, runs {_runs(bad)}"


def check_select_exact(gpu_idx, gpu_pooled32, keff, where="", reserved=None):
    """Top-k of the GPU's own fp32 pooled scores, from a CPU stable sort
    (reserved positions first, in position order, when a mask is given)."""
    P = np.asarray(gpu_pooled32, dtype=np.float32)
    check_finite(P, f"{where} pooled")
    if reserved is not None and reserved.any():
        rest = np.nonzero(~reserved)[0]
        order = np.concatenate([np.nonzero(reserved)[0], rest[np.argsort(-P[rest], kind="stable")]])
    else:
        order = np.argsort(-P, kind="stable")
    expect = np.sort(order[:keff])
    got = np.asarray(gpu_idx, dtype=np.int64)
    if not np.array_equal(got, expect):
        only_gpu = np.setdiff1d(got, expect)[:5]
        only_cpu = np.setdiff1d(expect, got)[:5]
        tau = P[order[keff - 1]] if keff else None
        raise AssertionError(f"{where}: selection differs from a stable sort of the GPU's pooled scores; "
                             f"k-th value {tau!r}; GPU-only {only_gpu.tolist()} -> {P[only_gpu].tolist() if len(only_gpu) and only_gpu.max() < len(P) else []}; "
                             f"CPU-only {only_cpu.tolist()} -> {P[only_cpu].tolist()}; "
                             f"GPU idx ascending: {bool(np.all(np.diff(got) > 0))}, in range: {bool(got.min() >= 0 and got.max() < len(P)) if len(got) else True}")


def segments(spec, out_offsets):
    """(b, h, L_b, score offset, out offset, keff) of every segment."""
    res = []
    key_off = 0
    for b, L in enumerate(spec.seq_lens):
        for h in range(spec.Hkv):
            s = b * spec.Hkv + h
            res.append((b, h, L, spec.Hkv * key_off + h * L, out_offsets[s], out_offsets[s + 1] - out_offsets[s]))
        key_off += L
    return res


def check_against_oracle(spec, case, out, ref, heads=None, scores=None):
    """Compare one compress() result with the oracle result for the given heads.

    ``out``: dict with idx, K_out, V_out, pooled (torch, GPU); ``ref``: oracle
    result dict; ``scores``: optional GPU unpooled scores.  Returns stats.
    """
    import torch

    idx = out["idx"].cpu().numpy()
    pooled = out["pooled"].cpu().numpy() if out.get("pooled") is not None else None
    Kc = case["K"].cpu()
    Vc = case["V"].cpu()
    Ko = out["K_out"].cpu()
    Vo = out["V_out"].cpu()
    sc = scores.cpu().numpy() if scores is not None else None
    starts = np.concatenate([[0], np.cumsum(spec.seq_lens)])
    stats = {"near_tie_diffs": 0, "max_rel": 0.0, "beyond_diag": 0, "segments": 0}
    for (b, h, L, soff, ooff, keff) in segments(spec, out["out_offsets"]):
        gidx = idx[ooff:ooff + keff]
        res = reserved_mask(L, getattr(spec, "sink", 0), getattr(spec, "recent", 0))
        # gathered rows are exact copies of the rows the GPU chose (all segments)
        if keff:
            rows = torch.from_numpy(starts[b] + gidx.astype(np.int64))
            assert torch.equal(Ko[ooff:ooff + keff], Kc[rows, h]), f"K_out mismatch in segment {(b, h)}"
            assert torch.equal(Vo[ooff:ooff + keff], Vc[rows, h]), f"V_out mismatch in segment {(b, h)}"
        if sc is not None:
            check_finite(sc[soff:soff + L], f"segment {(b, h)} scores")
        if pooled is not None:
            check_select_exact(gidx, pooled[soff:soff + L], keff, where=f"segment {(b, h)}", reserved=res)
        if heads is not None and (b, h) not in heads:
            continue
        r = ref[(b, h)]
        if pooled is not None:
            st = check_scores(pooled[soff:soff + L], r["pooled"], f"pooled{(b, h)}")
            stats["max_rel"] = max(stats["max_rel"], st["max_rel"])
            stats["beyond_diag"] += st["beyond_diag"]
        if sc is not None:
            check_scores(sc[soff:soff + L], r["scores"], f"scores{(b, h)}")
        stats["near_tie_diffs"] += check_selection(gidx, r["idx"], r["pooled"], keff, L, reserved=res)
        stats["segments"] += 1
    return stats
