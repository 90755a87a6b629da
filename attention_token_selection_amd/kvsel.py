"""Thin ctypes binding of libkvsel (include/kvsel.h).

The functions here only marshal arguments: they check that torch tensors
have the device, dtype, contiguity and size the problem implies (so a
mis-sized buffer is rejected on the host instead of faulting on the GPU),
take their data pointers and the current HIP stream, and call the C entry
point of the same name.  Every step of the computation runs in libkvsel's
kernels.  There is no fallback: if the library is missing, importing this
module raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvsel.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvsel.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python attention_token_selection_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

KVSEL_OK, KVSEL_EINVAL, KVSEL_EUNSUPPORTED, KVSEL_EHIP = 0, 1, 2, 3
POOLS = {"none": 0, "avg": 1, "max": 2}
WEIGHTINGS = {"alpha": 0, "exp": 1}
GQAS = {"sum": 0, "mean": 1}


class KvselProblem(ctypes.Structure):
    """Mirror of ``struct kvsel_problem``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("L", ctypes.c_int64),
        ("seq_offsets_h", ctypes.POINTER(ctypes.c_int64)),
        ("w", ctypes.c_int32),
        ("has_decode", ctypes.c_int32),
        ("alpha", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("pool", ctypes.c_int32),
        ("pool_kernel", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("budgets_h", ctypes.POINTER(ctypes.c_int32)),
        ("key_chunk", ctypes.c_int32),
        ("weighting", ctypes.c_int32),
        ("lambda_", ctypes.c_float),
        ("sink_tokens", ctypes.c_int32),
        ("recent_tokens", ctypes.c_int32),
        ("gqa", ctypes.c_int32),
        ("stream_keys", ctypes.c_int32),
    ]


_P = ctypes.POINTER(KvselProblem)
_vp = ctypes.c_void_p
_lib.kvsel_abi_version.restype = ctypes.c_int
_lib.kvsel_status_string.restype = ctypes.c_char_p
_lib.kvsel_status_string.argtypes = [ctypes.c_int]
_lib.kvsel_last_error.restype = ctypes.c_char_p
_lib.kvsel_plan.restype = ctypes.c_int
_lib.kvsel_plan.argtypes = [_P, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int64)]
_lib.kvsel_score.restype = ctypes.c_int
_lib.kvsel_score.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_row_stats.restype = ctypes.c_int
_lib.kvsel_row_stats.argtypes = [_P, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_score_from_stats.restype = ctypes.c_int
_lib.kvsel_score_from_stats.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_pool_topk.restype = ctypes.c_int
_lib.kvsel_pool_topk.argtypes = [_P, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_gather.restype = ctypes.c_int
_lib.kvsel_gather.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.kvsel_compress.restype = ctypes.c_int
_lib.kvsel_compress.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_compress_noalloc.restype = ctypes.c_int
_lib.kvsel_compress_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.kvsel_profile_layer.restype = ctypes.c_int
_lib.kvsel_profile_layer.argtypes = [_P, _vp, _vp, _vp, ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_tier_rank.restype = ctypes.c_int
_lib.kvsel_tier_rank.argtypes = [_P, _vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_topk_mass.restype = ctypes.c_int
_lib.kvsel_topk_mass.argtypes = [_P, _vp, ctypes.c_int32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.kvsel_allocate_budgets.restype = ctypes.c_int
_lib.kvsel_allocate_budgets.argtypes = [ctypes.c_int32, ctypes.c_int32, _vp, _vp, ctypes.c_int64, _vp]


class KvselError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.kvsel_last_error().decode()
        name = _lib.kvsel_status_string(status).decode()
        super().__init__(f"{where}: {name} ({status}): {detail}")


def _check(status: int, where: str):
    if status != KVSEL_OK:
        raise KvselError(status, where)


def exported_functions() -> list:
    """Names of the functions include/kvsel.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(kvsel_[a-z_]+)\s*\(", text)))


def abi_version() -> int:
    return _lib.kvsel_abi_version()


class Problem:
    """A kvsel_problem plus the host arrays it points to.

    ``seq_lens`` (list of prefix lengths) or ``L`` with ``batch``; a uniform
    ``k`` or ``budgets`` [B][Hkv]; ``pool`` is "none", "avg" or "max".
    """

    def __init__(self, *, Hq: int, Hkv: int, w: int, d: int = 128, seq_lens: Optional[Sequence[int]] = None,
                 L: int = 0, batch: int = 1, has_decode: bool = False, alpha: float = 0.0, causal: bool = True,
                 scale: float = 0.0, pool: str = "none", pool_kernel: int = 1, k: int = 0,
                 budgets=None, key_chunk: int = 0, weighting: str = "alpha", lam: float = 0.0, sink: int = 0,
                 recent: int = 0, gqa: str = "sum", stream_keys: int = 0):
        if seq_lens is None:
            seq_lens = [int(L)] * int(batch)
        self.seq_lens = [int(x) for x in seq_lens]
        self.Hq, self.Hkv, self.d, self.w = int(Hq), int(Hkv), int(d), int(w)
        self.has_decode = bool(has_decode)
        self.budgets = None if budgets is None else [[int(x) for x in row] for row in budgets]
        self.k = int(k)
        offs = [0]
        for x in self.seq_lens:
            offs.append(offs[-1] + x)
        self._offs = (ctypes.c_int64 * len(offs))(*offs)
        self._budgets = None
        if self.budgets is not None:
            flat = [x for row in self.budgets for x in row]
            self._budgets = (ctypes.c_int32 * max(1, len(flat)))(*flat)
        s = KvselProblem()
        s.batch = len(self.seq_lens)
        s.Hq, s.Hkv, s.d = self.Hq, self.Hkv, self.d
        s.L = self.seq_lens[0] if self.seq_lens else 0
        s.seq_offsets_h = ctypes.cast(self._offs, ctypes.POINTER(ctypes.c_int64))
        s.w = self.w
        s.has_decode = int(self.has_decode)
        s.alpha = float(alpha)
        s.causal = int(bool(causal))
        s.scale = float(scale)
        s.pool = POOLS[pool] if isinstance(pool, str) else int(pool)
        s.pool_kernel = int(pool_kernel)
        s.k = self.k
        s.budgets_h = ctypes.cast(self._budgets, ctypes.POINTER(ctypes.c_int32)) if self._budgets else None
        s.key_chunk = int(key_chunk)
        s.weighting = WEIGHTINGS[weighting] if isinstance(weighting, str) else int(weighting)
        s.lambda_ = float(lam)
        s.sink_tokens = int(sink)
        s.recent_tokens = int(recent)
        s.gqa = GQAS[gqa] if isinstance(gqa, str) else int(gqa)
        s.stream_keys = int(stream_keys)
        self.struct = s

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def rows(self) -> int:
        return self.w + int(self.has_decode)

    @property
    def total_keys(self) -> int:
        return sum(self.seq_lens)

    def ref(self):
        return ctypes.byref(self.struct)


def kvsel_plan(problem: Problem):
    """(workspace bytes, out_offsets list of B*Hkv+1 ints)."""
    ws = ctypes.c_size_t(0)
    n = problem.batch * problem.Hkv + 1
    offs = (ctypes.c_int64 * n)()
    _check(_lib.kvsel_plan(problem.ref(), ctypes.byref(ws), offs), "kvsel_plan")
    return int(ws.value), list(offs)


# ---------------------------------------------------------------- torch marshalling
def _torch():
    import torch

    return torch


def _ptr(t, name, dtype, numel, device=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _sizes(p: Problem):
    ws, offs = kvsel_plan(p)
    return {
        "Q": p.batch * p.rows * p.Hq * p.d,
        "K": p.total_keys * p.Hkv * p.d,
        "scores": p.total_keys * p.Hkv,
        "kept": offs[-1],
        "ws": ws,
        "offs": offs,
    }


def kvsel_score(problem: Problem, Q, K, scores, ws, stream=None):
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    args = (_ptr(Q, "Q", torch.bfloat16, n["Q"], dev), _ptr(K, "K", torch.bfloat16, n["K"], dev),
            _ptr(scores, "scores", torch.float32, n["scores"], dev), _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_score(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)), "kvsel_score")


def kvsel_row_stats(problem: Problem, Q, K, ws, stream=None):
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    args = (_ptr(Q, "Q", torch.bfloat16, n["Q"], dev), _ptr(K, "K", torch.bfloat16, n["K"], dev),
            _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_row_stats(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)),
               "kvsel_row_stats")


def kvsel_score_from_stats(problem: Problem, Q, K, scores, ws, stream=None):
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    args = (_ptr(Q, "Q", torch.bfloat16, n["Q"], dev), _ptr(K, "K", torch.bfloat16, n["K"], dev),
            _ptr(scores, "scores", torch.float32, n["scores"], dev), _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_score_from_stats(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)),
               "kvsel_score_from_stats")


def kvsel_pool_topk(problem: Problem, scores, pooled, idx, ws, stream=None):
    torch = _torch()
    n = _sizes(problem)
    dev = scores.device
    args = (_ptr(scores, "scores", torch.float32, n["scores"], dev),
            _ptr(pooled, "pooled", torch.float32, n["scores"], dev),
            _ptr(idx, "idx", torch.int32, n["kept"], dev) if n["kept"] else (idx.data_ptr() if idx is not None else None),
            _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_pool_topk(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)),
               "kvsel_pool_topk")


def kvsel_gather(problem: Problem, idx, K, V, K_out, V_out, stream=None):
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    kept = n["kept"]
    args = (_ptr(idx, "idx", torch.int32, kept, dev) if kept else None,
            _ptr(K, "K", torch.bfloat16, n["K"], dev), _ptr(V, "V", torch.bfloat16, n["K"], dev),
            _ptr(K_out, "K_out", torch.bfloat16, kept * problem.d, dev) if kept else None,
            _ptr(V_out, "V_out", torch.bfloat16, kept * problem.d, dev) if kept else None)
    with torch.cuda.device(dev):
        _check(_lib.kvsel_gather(problem.ref(), *args, _stream(stream, dev)), "kvsel_gather")


def kvsel_compress(problem: Problem, Q, K, V, idx, K_out, V_out, pooled, ws, stream=None):
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    kept = n["kept"]
    args = (_ptr(Q, "Q", torch.bfloat16, n["Q"], dev), _ptr(K, "K", torch.bfloat16, n["K"], dev),
            _ptr(V, "V", torch.bfloat16, n["K"], dev),
            _ptr(idx, "idx", torch.int32, kept, dev) if kept else None,
            _ptr(K_out, "K_out", torch.bfloat16, kept * problem.d, dev) if kept else None,
            _ptr(V_out, "V_out", torch.bfloat16, kept * problem.d, dev) if kept else None,
            _ptr(pooled, "pooled", torch.float32, n["scores"], dev),
            _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_compress(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)),
               "kvsel_compress")

def kvsel_compress_noalloc(problem: Problem, Q, K, V, idx, K_out, V_out, pooled, stream=None):
    """kvsel_compress with the library's own per-GPU scratch as workspace
    (no allocation; calls that overlap on one GPU race)."""
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    kept = n["kept"]
    args = (_ptr(Q, "Q", torch.bfloat16, n["Q"], dev), _ptr(K, "K", torch.bfloat16, n["K"], dev),
            _ptr(V, "V", torch.bfloat16, n["K"], dev),
            _ptr(idx, "idx", torch.int32, kept, dev) if kept else None,
            _ptr(K_out, "K_out", torch.bfloat16, kept * problem.d, dev) if kept else None,
            _ptr(V_out, "V_out", torch.bfloat16, kept * problem.d, dev) if kept else None,
            _ptr(pooled, "pooled", torch.float32, n["scores"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_compress_noalloc(problem.ref(), *args, _stream(stream, dev)), "kvsel_compress_noalloc")


def kvsel_profile_layer(problem: Problem, Q, K, profile, ws, accumulate: bool = False, stream=None):
    """One layer's contribution to the warm-up importance profile [sum L]."""
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    args = (_ptr(Q, "Q", torch.bfloat16, n["Q"], dev), _ptr(K, "K", torch.bfloat16, n["K"], dev),
            _ptr(profile, "profile", torch.float32, problem.total_keys, dev), ctypes.c_int32(int(accumulate)),
            _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_profile_layer(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)),
               "kvsel_profile_layer")


def kvsel_tier_rank(problem: Problem, profile, n_fast: int, n_mid: int, tier, ws, stream=None):
    """Three-tier labels (int8 [sum L]: 0 fast, 1 middle, 2 backing) from the profile."""
    torch = _torch()
    n = _sizes(problem)
    dev = profile.device
    args = (_ptr(profile, "profile", torch.float32, problem.total_keys, dev), ctypes.c_int64(int(n_fast)),
            ctypes.c_int64(int(n_mid)), _ptr(tier, "tier", torch.int8, problem.total_keys, dev),
            _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_tier_rank(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)),
               "kvsel_tier_rank")

def kvsel_topk_mass(problem: Problem, pooled, sizes, mass, ws, stream=None):
    """Kept importance of each candidate budget: mass [B*Hkv][len(sizes)] fp32."""
    torch = _torch()
    n = _sizes(problem)
    dev = pooled.device
    sz = (ctypes.c_int32 * len(sizes))(*[int(x) for x in sizes])
    args = (_ptr(pooled, "pooled", torch.float32, n["scores"], dev), ctypes.c_int32(len(sizes)),
            ctypes.cast(sz, ctypes.c_void_p),
            _ptr(mass, "mass", torch.float32, problem.batch * problem.Hkv * len(sizes), dev),
            _ptr(ws, "ws", torch.uint8, n["ws"], dev))
    with torch.cuda.device(dev):
        _check(_lib.kvsel_topk_mass(problem.ref(), *args, ctypes.c_size_t(ws.numel()), _stream(stream, dev)),
               "kvsel_topk_mass")


def kvsel_allocate_budgets(benefit, sizes, total: int):
    """Host-side greedy allocation: benefit [items][len(sizes)] -> budgets [items] (numpy int32)."""
    import numpy as np

    b = np.ascontiguousarray(benefit, dtype=np.float64)
    items, ns = b.shape
    if ns != len(sizes):
        raise ValueError("benefit needs one column per candidate size")
    sz = np.ascontiguousarray(sizes, dtype=np.int32)
    out = np.zeros(items, dtype=np.int32)
    _check(_lib.kvsel_allocate_budgets(items, ns, sz.ctypes.data, b.ctypes.data, int(total), out.ctypes.data),
           "kvsel_allocate_budgets")
    return out


def alloc_outputs(problem: Problem, device, pooled: bool = True):
    """Output tensors and workspace for kvsel_compress (torch.empty; the
    workspace needs no initialisation)."""
    torch = _torch()
    n = _sizes(problem)
    kept = n["kept"]
    return {
        "idx": torch.empty(max(kept, 1), dtype=torch.int32, device=device),
        "K_out": torch.empty(max(kept, 1), problem.d, dtype=torch.bfloat16, device=device),
        "V_out": torch.empty(max(kept, 1), problem.d, dtype=torch.bfloat16, device=device),
        "pooled": torch.empty(max(n["scores"], 1), dtype=torch.float32, device=device) if pooled else None,
        "ws": torch.empty(n["ws"], dtype=torch.uint8, device=device),
        "out_offsets": n["offs"],
    }


def compress(problem: Problem, Q, K, V, pooled: bool = True, stream=None):
    """Allocate outputs, run kvsel_compress, return them in a dict.  With a
    stream given, the outputs and workspace are allocated on that stream (so
    that torch's caching allocator ties their reuse to the work that writes
    them there)."""
    torch = _torch()
    if stream is None:
        out = alloc_outputs(problem, K.device, pooled=pooled)
    else:
        with torch.cuda.stream(stream):
            out = alloc_outputs(problem, K.device, pooled=pooled)
    kvsel_compress(problem, Q, K, V, out["idx"], out["K_out"], out["V_out"], out["pooled"], out["ws"], stream)
    return out


def bind_compress(problem: Problem, Q, K, V, idx, K_out, V_out, pooled, ws, stream=None):
    """Check the arguments once and return a callable that only re-issues the
    kvsel_compress C call with the same pointers (for tight loops and graph
    capture, where per-call Python checks would dominate)."""
    torch = _torch()
    n = _sizes(problem)
    dev = K.device
    kept = n["kept"]
    args = (problem.ref(), _ptr(Q, "Q", torch.bfloat16, n["Q"], dev), _ptr(K, "K", torch.bfloat16, n["K"], dev),
            _ptr(V, "V", torch.bfloat16, n["K"], dev),
            _ptr(idx, "idx", torch.int32, kept, dev) if kept else None,
            _ptr(K_out, "K_out", torch.bfloat16, kept * problem.d, dev) if kept else None,
            _ptr(V_out, "V_out", torch.bfloat16, kept * problem.d, dev) if kept else None,
            _ptr(pooled, "pooled", torch.float32, n["scores"], dev),
            _ptr(ws, "ws", torch.uint8, n["ws"], dev), ctypes.c_size_t(ws.numel()), _stream(stream, dev))
    fn = _lib.kvsel_compress
    keep = (problem, Q, K, V, idx, K_out, V_out, pooled, ws, stream)

    def call():
        _ = keep  # the tensors must outlive the bound call
        st = fn(*args)
        if st != KVSEL_OK:
            raise KvselError(st, "kvsel_compress")

    return call
