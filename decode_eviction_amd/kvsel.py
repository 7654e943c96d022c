"""Thin ctypes binding of libkvsel (include/kvsel.h).

Functions carry the C names.  They only marshal arguments: device pointers
and shapes come from torch tensors, the stream is torch's current stream
unless one is given, and the workspace is a torch uint8 tensor the binding
allocates when the caller passes none.  Every step of the computation runs in
the HIP kernels of libkvsel.so; if the library is missing this module raises
instead of computing anything itself.

Streams: every tensor the binding allocates (outputs, zero-filled compacted
caches, the workspace) is allocated and filled on the stream the kernels run
on, inside ``torch.cuda.stream(s)``, so the fills are ordered before the
kernels and the caching allocator does not reuse a temporary workspace
before the kernels on ``s`` are done with it.  Tensors the caller passes are
the caller's to order, as with any torch operation on a side stream.

Arguments are checked before the call: device, contiguity, element types
(lengths int32 with at least b entries, q/v of k's dtype) and the shapes and
dtypes of caller-given outputs; a mismatch raises ValueError or TypeError.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the library to load: $KVSEL_LIB when set (for instance the debug build,
# decode_eviction_amd/libkvsel_debug.so), else the in-tree libkvsel.so
LIB_PATH = os.environ.get("KVSEL_LIB") or os.path.join(_HERE, "libkvsel.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "kvsel.h")

KVSEL_OK, KVSEL_ERR_INVALID_ARG, KVSEL_ERR_UNSUPPORTED, KVSEL_ERR_WORKSPACE, KVSEL_ERR_HIP = range(5)
KVSEL_BF16, KVSEL_F32 = 0, 1
KVSEL_R_GRAM, KVSEL_R_KEYSUM = 0, 1
MODES = {"gram": KVSEL_R_GRAM, "keysum": KVSEL_R_KEYSUM}

_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "kvsel_status_string": (ctypes.c_char_p, [_I]),
    "kvsel_score_evict_workspace": (_S, [_I] * 7),
    "kvsel_scores": (_I, [_I, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _S, _P]),
    "kvsel_select_workspace": (_S, [_I, _I, _I]),
    "kvsel_select_topb": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _S, _P]),
    "kvsel_select_topb_heads": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _S, _P]),
    "kvsel_gather": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P]),
    "kvsel_score_evict": (_I, [_I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                               _P, _P, _I, _P, _P, _P, _S, _P]),
    "kvsel_score_evict_static": (_I, [_I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                      _P, _P, _I, _P, _P, _P]),
    "kvsel_score_evict_heads": (_I, [_I, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                     _P, _P, _I, _P, _P, _P, _S, _P]),
    "kvsel_score_evict_heads_traced": (_I, [_I, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                            _F, _I, _P, _P, _I, _P, _P, _P, _S, _P, _P, _I]),
    "kvsel_score_evict_traced": (_I, [_I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                      _P, _P, _I, _P, _P, _P, _S, _P, _P, _I]),
    "kvsel_select_evict_slots": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _P, _P, _S, _P]),
    "kvsel_score_evict_slots": (_I, [_I, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                                     _P, _I, _P, _P, _P, _S, _P]),
    "kvsel_score_evict_slots_traced": (_I, [_I, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                            _F, _I, _P, _I, _P, _P, _P, _S, _P, _P, _I]),
    "kvsel_slots_write": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _P]),
    "kvsel_threshold_cut_workspace": (_S, [_I] * 5),
    "kvsel_threshold_cut_traced": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P,
                                        _P, _S, _P, _P, _I]),
    "kvsel_threshold_cut": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P,
                                 _P, _S, _P]),
    "kvsel_threshold_cut_from_attn": (_I, [_P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _S, _P]),
    "kvsel_threshold_cut_rows_workspace": (_S, [_I] * 6),
    "kvsel_threshold_cut_rows": (_I, [_I, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                      _F, _P, _P, _P, _I, _P, _S, _P]),
    "kvsel_threshold_cut_rows_traced": (_I, [_I, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                             _I, _F, _P, _P, _P, _I, _P, _S, _P, _P, _I]),
    "kvsel_cut_compact": (_I, [_I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P]),
    "kvsel_workspace_error": (_I, [_P, _P, _P]),
}

_lib = None


class KvselError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libkvsel.so (built in-tree by decode_eviction_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_eviction_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/kvsel.h declares."""
    with open(HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(kvsel_\w+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().kvsel_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != KVSEL_OK:
        raise KvselError(fn, status)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KVSEL_BF16
    if t.dtype == torch.float32:
        return KVSEL_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_of(stream):
    return stream if stream is not None else torch.cuda.current_stream()


def _handle(s):
    return ctypes.c_void_p(s.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _need_lengths(lengths, b):
    if lengths.dtype != torch.int32:
        raise TypeError(f"lengths must be int32, got {lengths.dtype}")
    if lengths.numel() < b:
        raise ValueError(f"lengths has {lengths.numel()} entries for {b} sequences")


def _need_i32(t, name, numel=None, shape=None):
    if t is None:
        return
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} entries, needs {numel}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, needs {tuple(shape)}")


def _need_like(ref, name, t):
    """t (nullable) has ref's dtype (q and v against k)."""
    if t is not None and t.dtype != ref.dtype:
        raise TypeError(f"{name} is {t.dtype} but k is {ref.dtype}")


def _need_out(t, name, dtype, lead, min_rows=None, rows=None, tail=None):
    """Caller-given output: dtype, leading dims lead, then (rows[, tail])."""
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    sh = tuple(t.shape)
    want_nd = len(lead) + 1 + (1 if tail is not None else 0)
    if len(sh) != want_nd or sh[:len(lead)] != tuple(lead):
        raise ValueError(f"{name} has shape {sh}, needs leading dims {tuple(lead)} and {want_nd} dims")
    if tail is not None and sh[-1] != tail:
        raise ValueError(f"{name} has last dim {sh[-1]}, needs {tail}")
    r = sh[len(lead)]
    if rows is not None and r != rows:
        raise ValueError(f"{name} has {r} rows per head, needs {rows}")
    if min_rows is not None and r < min_rows:
        raise ValueError(f"{name} has {r} rows per head, needs at least {min_rows}")


def _workspace(nbytes: int, device, workspace):
    """Caller's workspace, or a new one (allocate inside the launch stream's context)."""
    if workspace is not None:
        if workspace.dtype != torch.uint8:
            raise TypeError("workspace must be a uint8 tensor")
        return workspace
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ R-KV

def kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, budget) -> int:
    return int(lib().kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, budget))


def _rkv_inputs(q_window, k, v, lengths):
    """Checks of the R-KV inputs; returns (b, hq, w, d, hkv, cap)."""
    _need_cuda(q_window, k, v, lengths)
    if q_window.dim() != 4 or k.dim() != 4:
        raise ValueError("q_window must be [b][Hq][w][d] and k [b][Hkv][cap][d]")
    b, hq, w, d = q_window.shape
    bk, hkv, cap, dk = k.shape
    if bk != b or dk != d:
        raise ValueError(f"k has shape {tuple(k.shape)} for q_window {tuple(q_window.shape)}")
    _dtype(k)
    _need_like(k, "q_window", q_window)
    _need_like(k, "v", v)
    if v is not None and tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v has shape {tuple(v.shape)}, k {tuple(k.shape)}")
    _need_lengths(lengths, b)
    return b, hq, w, d, hkv, cap


def kvsel_scores(q_window, k, lengths, lam=0.1, mode="gram", i_out=None, r_out=None, z_out=None,
                 workspace=None, stream=None):
    """I, R, Z (fp32 [b][Hkv][cap]) for q_window [b][Hq][w][d], k [b][Hkv][cap][d]."""
    b, hq, w, d, hkv, cap = _rkv_inputs(q_window, k, None, lengths)
    _need_cuda(i_out, r_out, z_out)
    for name, t in (("i_out", i_out), ("r_out", r_out), ("z_out", z_out)):
        _need_out(t, name, torch.float32, (b, hkv), rows=cap)
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if z_out is None:
            z_out = torch.empty((b, hkv, cap), dtype=torch.float32, device=k.device)
        ws = _workspace(kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, 1), k.device, workspace)
        st = lib().kvsel_scores(_dtype(k), MODES[mode], _ptr(q_window), _ptr(k), _ptr(lengths),
                                b, hq, hkv, d, w, cap, float(lam), _ptr(i_out), _ptr(r_out),
                                _ptr(z_out), _ptr(ws), ws.numel(), _handle(s))
    _check("kvsel_scores", st)
    return i_out, r_out, z_out


def kvsel_select_workspace(b, hkv, cap) -> int:
    return int(lib().kvsel_select_workspace(b, hkv, cap))


def _select_inputs(z, lengths):
    _need_cuda(z, lengths)
    if z.dtype != torch.float32 or z.dim() != 3:
        raise TypeError("z must be a float32 [b][Hkv][cap] tensor")
    b, hkv, cap = z.shape
    _need_lengths(lengths, b)
    return b, hkv, cap


def kvsel_select_topb(z, lengths, budget, idx_out=None, workspace=None, stream=None):
    b, hkv, cap = _select_inputs(z, lengths)
    _need_cuda(idx_out)
    _need_out(idx_out, "idx_out", torch.int32, (b, hkv), rows=budget)
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if idx_out is None:
            idx_out = torch.empty((b, hkv, budget), dtype=torch.int32, device=z.device)
        ws = _workspace(kvsel_select_workspace(b, hkv, cap), z.device, workspace)
        st = lib().kvsel_select_topb(_ptr(z), _ptr(lengths), b, hkv, cap, int(budget),
                                     _ptr(idx_out), _ptr(ws), ws.numel(), _handle(s))
    _check("kvsel_select_topb", st)
    return idx_out


def kvsel_select_topb_heads(z, lengths, budgets, budget_max, idx_out=None, workspace=None,
                            stream=None):
    """Top-budget per KV head with budgets [Hkv] (int32 device tensor)."""
    b, hkv, cap = _select_inputs(z, lengths)
    _need_cuda(budgets, idx_out)
    _need_i32(budgets, "budgets", numel=hkv)
    _need_out(idx_out, "idx_out", torch.int32, (b, hkv), rows=budget_max)
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if idx_out is None:
            idx_out = torch.empty((b, hkv, budget_max), dtype=torch.int32, device=z.device)
        ws = _workspace(kvsel_select_workspace(b, hkv, cap), z.device, workspace)
        st = lib().kvsel_select_topb_heads(_ptr(z), _ptr(lengths), _ptr(budgets), b, hkv, cap,
                                           int(budget_max), _ptr(idx_out), _ptr(ws), ws.numel(),
                                           _handle(s))
    _check("kvsel_select_topb_heads", st)
    return idx_out


def kvsel_gather(k, v, idx, k_out=None, v_out=None, stream=None):
    _need_cuda(k, v, idx, k_out, v_out)
    if k.dim() != 4:
        raise ValueError("k must be [b][Hkv][cap][d]")
    b, hkv, cap, d = k.shape
    _dtype(k)
    _need_like(k, "v", v)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v has shape {tuple(v.shape)}, k {tuple(k.shape)}")
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (b, hkv):
        raise ValueError(f"idx must be [b][Hkv][budget], got {tuple(idx.shape)}")
    _need_i32(idx, "idx")
    budget = idx.shape[2]
    _need_out(k_out, "k_out", k.dtype, (b, hkv), min_rows=budget, tail=d)
    _need_out(v_out, "v_out", k.dtype, (b, hkv), min_rows=budget, tail=d)
    if k_out is not None and v_out is not None and k_out.shape != v_out.shape:
        raise ValueError("k_out and v_out differ in shape")
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if k_out is None:
            k_out = torch.zeros((b, hkv, budget, d), dtype=k.dtype, device=k.device)
        if v_out is None:
            v_out = torch.zeros(tuple(k_out.shape), dtype=v.dtype, device=v.device)
        st = lib().kvsel_gather(_dtype(k), _ptr(k), _ptr(v), _ptr(idx), b, hkv, d, cap, budget,
                                _ptr(k_out), _ptr(v_out), k_out.shape[2], _handle(s))
    _check("kvsel_gather", st)
    return k_out, v_out


def _evict_outputs(k, b, hkv, d, budget, k_out, v_out, idx_out, scores_out, cap):
    _need_cuda(k_out, v_out, idx_out, scores_out)
    _need_out(k_out, "k_out", k.dtype, (b, hkv), min_rows=budget, tail=d)
    _need_out(v_out, "v_out", k.dtype, (b, hkv), min_rows=budget, tail=d)
    if k_out is not None and v_out is not None and k_out.shape != v_out.shape:
        raise ValueError("k_out and v_out differ in shape")
    _need_out(idx_out, "idx_out", torch.int32, (b, hkv), rows=budget)
    _need_out(scores_out, "scores_out", torch.float32, (b, hkv), rows=cap)


def kvsel_score_evict(q_window, k, v, lengths, budget, lam=0.1, mode="gram", k_out=None,
                      v_out=None, idx_out=None, scores_out=None, workspace=None, stream=None):
    """The whole step; returns (k_out, v_out, idx_out)."""
    b, hq, w, d, hkv, cap = _rkv_inputs(q_window, k, v, lengths)
    _evict_outputs(k, b, hkv, d, budget, k_out, v_out, idx_out, scores_out, cap)
    dev = k.device
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if k_out is None:
            k_out = torch.zeros((b, hkv, budget, d), dtype=k.dtype, device=dev)
        if v_out is None:
            v_out = torch.zeros(tuple(k_out.shape), dtype=v.dtype, device=dev)
        if idx_out is None:
            idx_out = torch.empty((b, hkv, budget), dtype=torch.int32, device=dev)
        ws = _workspace(kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, budget), dev, workspace)
        st = lib().kvsel_score_evict(_dtype(k), MODES[mode], _ptr(q_window), _ptr(k), _ptr(v),
                                     _ptr(lengths), b, hq, hkv, d, w, cap, float(lam), int(budget),
                                     _ptr(k_out), _ptr(v_out), k_out.shape[2], _ptr(idx_out),
                                     _ptr(scores_out), _ptr(ws), ws.numel(), _handle(s))
    _check("kvsel_score_evict", st)
    return k_out, v_out, idx_out


STATIC_SCRATCH_BYTES = 16 << 20   # KVSEL_STATIC_SCRATCH_BYTES


def kvsel_score_evict_static(q_window, k, v, lengths, budget, lam=0.1, mode="gram", k_out=None,
                             v_out=None, idx_out=None, scores_out=None, stream=None):
    """The whole step in the library's own device scratch array (no
    workspace); returns (k_out, v_out, idx_out).  Outputs not given are
    allocated here; pass all three to keep the call free of allocations."""
    b, hq, w, d, hkv, cap = _rkv_inputs(q_window, k, v, lengths)
    _evict_outputs(k, b, hkv, d, budget, k_out, v_out, idx_out, scores_out, cap)
    dev = k.device
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if k_out is None:
            k_out = torch.zeros((b, hkv, budget, d), dtype=k.dtype, device=dev)
        if v_out is None:
            v_out = torch.zeros(tuple(k_out.shape), dtype=v.dtype, device=dev)
        if idx_out is None:
            idx_out = torch.empty((b, hkv, budget), dtype=torch.int32, device=dev)
        st = lib().kvsel_score_evict_static(_dtype(k), MODES[mode], _ptr(q_window), _ptr(k),
                                            _ptr(v), _ptr(lengths), b, hq, hkv, d, w, cap,
                                            float(lam), int(budget), _ptr(k_out), _ptr(v_out),
                                            k_out.shape[2], _ptr(idx_out), _ptr(scores_out),
                                            _handle(s))
    _check("kvsel_score_evict_static", st)
    return k_out, v_out, idx_out


def kvsel_score_evict_heads(q_window, k, v, lengths, budgets, budget_max, lam=0.1, mode="gram",
                            k_out=None, v_out=None, idx_out=None, scores_out=None,
                            workspace=None, stream=None):
    """The whole step with per-head budgets; returns (k_out, v_out, idx_out)."""
    b, hq, w, d, hkv, cap = _rkv_inputs(q_window, k, v, lengths)
    _need_cuda(budgets)
    _need_i32(budgets, "budgets", numel=hkv)
    _evict_outputs(k, b, hkv, d, budget_max, k_out, v_out, idx_out, scores_out, cap)
    dev = k.device
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if k_out is None:
            k_out = torch.zeros((b, hkv, budget_max, d), dtype=k.dtype, device=dev)
        if v_out is None:
            v_out = torch.zeros(tuple(k_out.shape), dtype=v.dtype, device=dev)
        if idx_out is None:
            idx_out = torch.empty((b, hkv, budget_max), dtype=torch.int32, device=dev)
        ws = _workspace(kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, budget_max), dev,
                        workspace)
        st = lib().kvsel_score_evict_heads(_dtype(k), MODES[mode], _ptr(q_window), _ptr(k),
                                           _ptr(v), _ptr(lengths), _ptr(budgets), b, hq, hkv, d, w,
                                           cap, float(lam), int(budget_max), _ptr(k_out),
                                           _ptr(v_out), k_out.shape[2], _ptr(idx_out),
                                           _ptr(scores_out), _ptr(ws), ws.numel(), _handle(s))
    _check("kvsel_score_evict_heads", st)
    return k_out, v_out, idx_out


# ------------------------------------------------------------------ slot reuse

def _slot_outputs(b, hkv, cap, pos, budgets, evict_out, n_evict_out):
    _need_cuda(pos, budgets, evict_out, n_evict_out)
    _need_i32(pos, "pos", shape=(b, hkv, cap))
    _need_i32(budgets, "budgets", numel=hkv)
    _need_out(evict_out, "evict_out", torch.int32, (b, hkv))
    _need_i32(n_evict_out, "n_evict_out", shape=(b, hkv))


def kvsel_select_evict_slots(z, lengths, budget, pos=None, budgets=None, evict_out=None,
                             n_evict_out=None, workspace=None, stream=None):
    """Evicted slots (ascending, -1 padded) and their count per (sequence, KV head)."""
    b, hkv, cap = _select_inputs(z, lengths)
    _slot_outputs(b, hkv, cap, pos, budgets, evict_out, n_evict_out)
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if evict_out is None:
            evict_out = torch.empty((b, hkv, cap), dtype=torch.int32, device=z.device)
        if n_evict_out is None:
            n_evict_out = torch.empty((b, hkv), dtype=torch.int32, device=z.device)
        ws = _workspace(kvsel_select_workspace(b, hkv, cap), z.device, workspace)
        st = lib().kvsel_select_evict_slots(_ptr(z), _ptr(lengths), _ptr(pos), _ptr(budgets), b,
                                            hkv, cap, int(budget), _ptr(evict_out),
                                            evict_out.shape[2], _ptr(n_evict_out), _ptr(ws),
                                            ws.numel(), _handle(s))
    _check("kvsel_select_evict_slots", st)
    return evict_out, n_evict_out


def kvsel_score_evict_slots(q_window, k, lengths, budget, lam=0.1, mode="gram", pos=None,
                            budgets=None, evict_out=None, n_evict_out=None, scores_out=None,
                            workspace=None, stream=None):
    """Scores and evicted slots in one call; returns (evict_out, n_evict_out)."""
    b, hq, w, d, hkv, cap = _rkv_inputs(q_window, k, None, lengths)
    _slot_outputs(b, hkv, cap, pos, budgets, evict_out, n_evict_out)
    _need_cuda(scores_out)
    _need_out(scores_out, "scores_out", torch.float32, (b, hkv), rows=cap)
    dev = k.device
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if evict_out is None:
            evict_out = torch.empty((b, hkv, cap), dtype=torch.int32, device=dev)
        if n_evict_out is None:
            n_evict_out = torch.empty((b, hkv), dtype=torch.int32, device=dev)
        ws = _workspace(kvsel_score_evict_workspace(b, hq, hkv, d, w, cap, budget), dev, workspace)
        st = lib().kvsel_score_evict_slots(_dtype(k), MODES[mode], _ptr(q_window), _ptr(k),
                                           _ptr(lengths), _ptr(pos), _ptr(budgets), b, hq, hkv, d,
                                           w, cap, float(lam), int(budget), _ptr(evict_out),
                                           evict_out.shape[2], _ptr(n_evict_out),
                                           _ptr(scores_out), _ptr(ws), ws.numel(), _handle(s))
    _check("kvsel_score_evict_slots", st)
    return evict_out, n_evict_out


def kvsel_slots_write(k, v, k_new, v_new, evict, n_evict, pos=None, pos_new=None, stream=None):
    """Copy new tokens [b][Hkv][count][d] into the evicted slots of k/v (in place)."""
    _need_cuda(k, v, k_new, v_new, evict, n_evict, pos, pos_new)
    if k.dim() != 4 or k_new.dim() != 4:
        raise ValueError("k must be [b][Hkv][cap][d] and k_new [b][Hkv][count][d]")
    b, hkv, cap, d = k.shape
    _dtype(k)
    for name, t in (("v", v), ("k_new", k_new), ("v_new", v_new)):
        _need_like(k, name, t)
    if tuple(v.shape) != tuple(k.shape) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("v / v_new must have the shapes of k / k_new")
    if tuple(k_new.shape[:2]) != (b, hkv) or k_new.shape[3] != d:
        raise ValueError(f"k_new has shape {tuple(k_new.shape)} for k {tuple(k.shape)}")
    if evict.dim() != 3 or tuple(evict.shape[:2]) != (b, hkv):
        raise ValueError(f"evict must be [b][Hkv][stride], got {tuple(evict.shape)}")
    _need_i32(evict, "evict")
    _need_i32(n_evict, "n_evict", shape=(b, hkv))
    _need_i32(pos, "pos", shape=(b, hkv, cap))
    _need_i32(pos_new, "pos_new", numel=b)
    count = k_new.shape[2]
    s = _stream_of(stream)
    st = lib().kvsel_slots_write(_dtype(k), _ptr(k), _ptr(v), _ptr(pos), _ptr(k_new), _ptr(v_new),
                                 _ptr(pos_new), _ptr(evict), evict.shape[2], _ptr(n_evict), b, hkv,
                                 d, cap, count, _handle(s))
    _check("kvsel_slots_write", st)


# ------------------------------------------------------------------ ReFreeKV

def kvsel_threshold_cut_workspace(b, hq, hkv, d, cap) -> int:
    return int(lib().kvsel_threshold_cut_workspace(b, hq, hkv, d, cap))


def _cut_inputs(q, k, lengths, nd):
    _need_cuda(q, k, lengths)
    if q.dim() != nd or k.dim() != 4:
        raise ValueError("q must be [b][Hq](" + ("[k]" if nd == 4 else "") + ")[d], k [b][Hkv][cap][d]")
    b, hkv, cap, d = k.shape
    if q.shape[0] != b or q.shape[-1] != d:
        raise ValueError(f"q has shape {tuple(q.shape)} for k {tuple(k.shape)}")
    _dtype(k)
    _need_like(k, "q", q)
    _need_lengths(lengths, b)
    return b, q.shape[1], hkv, cap, d


def kvsel_threshold_cut(q_last, k, lengths, layer, n_full_layers=2, n_sink=4, T=0.01,
                        kept_out=None, workspace=None, stream=None):
    """Kept length per (sequence, KV head), int32 [b][Hkv]."""
    b, hq, hkv, cap, d = _cut_inputs(q_last, k, lengths, 3)
    _need_cuda(kept_out)
    _need_i32(kept_out, "kept_out", shape=(b, hkv))
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if kept_out is None:
            kept_out = torch.empty((b, hkv), dtype=torch.int32, device=k.device)
        ws = _workspace(kvsel_threshold_cut_workspace(b, hq, hkv, d, cap), k.device, workspace)
        st = lib().kvsel_threshold_cut(_dtype(k), _ptr(q_last), _ptr(k), _ptr(lengths), b, hq,
                                       hkv, d, cap, int(layer), int(n_full_layers), int(n_sink),
                                       float(T), _ptr(kept_out), _ptr(ws), ws.numel(), _handle(s))
    _check("kvsel_threshold_cut", st)
    return kept_out


def kvsel_threshold_cut_rows_workspace(b, hq, hkv, d, cap, k_rows) -> int:
    return int(lib().kvsel_threshold_cut_rows_workspace(b, hq, hkv, d, cap, k_rows))


def kvsel_threshold_cut_rows(q_rows, k, lengths, layer, n_full_layers=2, n_sink=4, T=0.01,
                             v=None, k_out=None, v_out=None, kept_out=None, workspace=None,
                             stream=None):
    """Kept length per (sequence, KV head) from the last k rows, q_rows
    [b][Hq][k][d]; with v and k_out/v_out also the sink + suffix compaction."""
    b, hq, hkv, cap, d = _cut_inputs(q_rows, k, lengths, 4)
    k_rows = q_rows.shape[2]
    _need_cuda(v, k_out, v_out, kept_out)
    _need_like(k, "v", v)
    if v is not None and tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v has shape {tuple(v.shape)}, k {tuple(k.shape)}")
    _need_out(k_out, "k_out", k.dtype, (b, hkv), min_rows=cap, tail=d)
    _need_out(v_out, "v_out", k.dtype, (b, hkv), min_rows=cap, tail=d)
    if k_out is not None and v_out is not None and k_out.shape != v_out.shape:
        raise ValueError("k_out and v_out differ in shape")
    _need_i32(kept_out, "kept_out", shape=(b, hkv))
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if kept_out is None:
            kept_out = torch.empty((b, hkv), dtype=torch.int32, device=k.device)
        ws = _workspace(kvsel_threshold_cut_rows_workspace(b, hq, hkv, d, cap, k_rows), k.device,
                        workspace)
        st = lib().kvsel_threshold_cut_rows(_dtype(k), _ptr(q_rows), k_rows, _ptr(k), _ptr(v),
                                            _ptr(lengths), b, hq, hkv, d, cap, int(layer),
                                            int(n_full_layers), int(n_sink), float(T),
                                            _ptr(kept_out), _ptr(k_out), _ptr(v_out),
                                            0 if k_out is None else k_out.shape[2], _ptr(ws),
                                            ws.numel(), _handle(s))
    _check("kvsel_threshold_cut_rows", st)
    return kept_out


def kvsel_cut_compact(k, v, lengths, kept_len, n_sink=4, k_out=None, v_out=None, stream=None):
    """Sink + suffix compaction from given kept lengths; returns (k_out, v_out)."""
    _need_cuda(k, v, lengths, kept_len, k_out, v_out)
    if k.dim() != 4:
        raise ValueError("k must be [b][Hkv][cap][d]")
    b, hkv, cap, d = k.shape
    _dtype(k)
    _need_like(k, "v", v)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v has shape {tuple(v.shape)}, k {tuple(k.shape)}")
    _need_lengths(lengths, b)
    _need_i32(kept_len, "kept_len", shape=(b, hkv))
    _need_out(k_out, "k_out", k.dtype, (b, hkv), tail=d)
    _need_out(v_out, "v_out", k.dtype, (b, hkv), tail=d)
    if k_out is not None and v_out is not None and k_out.shape != v_out.shape:
        raise ValueError("k_out and v_out differ in shape")
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if k_out is None:
            k_out = torch.zeros_like(k)
        if v_out is None:
            v_out = torch.zeros(tuple(k_out.shape), dtype=v.dtype, device=v.device)
        st = lib().kvsel_cut_compact(_dtype(k), _ptr(k), _ptr(v), _ptr(lengths), _ptr(kept_len),
                                     b, hkv, d, cap, int(n_sink), _ptr(k_out), _ptr(v_out),
                                     k_out.shape[2], _handle(s))
    _check("kvsel_cut_compact", st)
    return k_out, v_out


def kvsel_threshold_cut_from_attn(attn_last, lengths, hkv, n_sink=4, T=0.01, kept_out=None,
                                  workspace=None, stream=None):
    _need_cuda(attn_last, lengths, kept_out)
    if attn_last.dtype != torch.float32 or attn_last.dim() != 3:
        raise TypeError("attn_last must be a float32 [b][Hq][cap] tensor")
    b, hq, cap = attn_last.shape
    _need_lengths(lengths, b)
    _need_i32(kept_out, "kept_out", shape=(b, hkv))
    s = _stream_of(stream)
    with torch.cuda.stream(s):
        if kept_out is None:
            kept_out = torch.empty((b, hkv), dtype=torch.int32, device=attn_last.device)
        ws = _workspace(kvsel_threshold_cut_workspace(b, hq, hkv, 64, cap), attn_last.device,
                        workspace)
        st = lib().kvsel_threshold_cut_from_attn(_ptr(attn_last), _ptr(lengths), b, hq, hkv, cap,
                                                 int(n_sink), float(T), _ptr(kept_out), _ptr(ws),
                                                 ws.numel(), _handle(s))
    _check("kvsel_threshold_cut_from_attn", st)
    return kept_out


def kvsel_workspace_error(workspace, stream=None) -> int:
    flag = ctypes.c_int32(0)
    st = lib().kvsel_workspace_error(_ptr(workspace), ctypes.byref(flag), _handle(_stream_of(stream)))
    _check("kvsel_workspace_error", st)
    return int(flag.value)
