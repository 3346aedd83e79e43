"""Speculative verify-and-accept and the P-EAGLE draft batch on MI355X.

Thin Python binding over ``libspecverify.so`` (C ABI in include/spec_verify.h).
The functions here only marshal arguments: they check tensor shapes, dtypes
and devices, allocate outputs with torch when the caller passes none, and call
the library on the current HIP stream.  All computation runs in the library's
HIP kernels; there is no other implementation to fall back to, and every call
raises if the library is missing or returns an error.

One decode round, with the drafter's distributions handed over as its logits
and row descriptors (tensors on the GPU; shapes as in the C header)::

    tok, _, desc = spec_draft_sample(drafter_logits, K, T, uniforms=u_draft,
                                     row_index=sample_rows, want_draft_probs=False,
                                     want_row_desc=True)
    out, acc, _ = spec_verify_sample_lq(target_logits, drafter_logits, desc, tok,
                                        u_verify, T, drafter_rows=sample_rows)
    batch = peagle_build_draft_batch(out, acc, tok, start_pos, block_table,
                                     block_size, target_hidden, h_shared, mask_id)

spec_verify_greedy / spec_verify_sample / spec_verify_mixed take a dense q
instead; spec_verify_tree verifies draft trees; StepGraph captures a verify,
build and acceptance-metrics step as one HIP graph.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

__all__ = [
    "require_library", "library_path", "sv_status_string", "spec_verify_workspace_bytes",
    "spec_verify_greedy", "spec_verify_sample", "peagle_build_draft_batch",
    "SpecVerifyError", "SV_F32", "SV_BF16", "SV_F16", "PADDING_SLOT_ID",
    "spec_verify_mixed", "spec_verify_sample_lq", "spec_verify_mixed_lq",
    "spec_verify_sample_noalloc", "spec_verify_greedy_early_exit",
    "spec_verify_sample_early_exit", "spec_verify_mixed_early_exit",
    "spec_verify_sample_lq_early_exit", "spec_verify_mixed_lq_early_exit",
    "spec_verify_tree_early_exit", "spec_verify_tree_lq_early_exit", "spec_verify_tree_mixed",
    "spec_verify_tree_mixed_early_exit",
    "noalloc_scratch_bytes", "spec_verify_tree", "spec_verify_tree_lq", "spec_draft_sample",
    "spec_accept_metrics", "accept_metrics_buffer", "acceptance_summary", "StepGraph",
    "trace_begin", "trace_read", "trace_end",
    "DEVERR_DRAFT_TOKEN", "DEVERR_ACCEPT_COUNT", "DEVERR_BLOCK_TABLE",
]

SV_F32, SV_BF16, SV_F16 = 0, 1, 2
PADDING_SLOT_ID = -1
DEVERR_DRAFT_TOKEN, DEVERR_ACCEPT_COUNT, DEVERR_BLOCK_TABLE = 1, 2, 4
DEVERR_ROW_INDEX, DEVERR_TEMPERATURE, DEVERR_TREE = 8, 16, 32
MAX_B, MAX_K, MAX_V = 1 << 20, 63, 1 << 19      # SV_MAX_B, SV_MAX_K, SV_MAX_V

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspecverify.so")
_lib = None
_lock = threading.Lock()

_p = ctypes.c_void_p
_i = ctypes.c_int
_SIGS = {
    "sv_status_string": (ctypes.c_char_p, [_i]),
    "spec_verify_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i]),
    "spec_verify_greedy": (_i, [_p, _i, _p, _i, _i, _i, _p, _p, _p, ctypes.c_size_t, _p, _p]),
    "spec_verify_sample": (_i, [_p, _i, _p, _p, _p, ctypes.c_float, _i, _i, _i, _p, _p, _p, _p,
                                ctypes.c_size_t, _p, _p]),
    "peagle_build_draft_batch": (_i, [_p, _p, _p, _p, _p, _i, _i, _p, _p, _i, ctypes.c_int32,
                                      _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]),
    "spec_verify_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "spec_verify_sample_noalloc": (_i, [_p, _i, _p, _p, _p, ctypes.c_float, _i, _i, _i, _p, _p,
                                        _p, _p, _p]),
    "spec_verify_mixed": (_i, [_p, _i, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p,
                               ctypes.c_size_t, _p, _p]),
    "spec_verify_greedy_early_exit": (_i, [_p, _i, _p, _i, _i, _i, _p, _p, _p, ctypes.c_size_t,
                                           _p, _p]),
    "spec_verify_sample_early_exit": (_i, [_p, _i, _p, _p, _p, ctypes.c_float, _i, _i, _i, _p,
                                           _p, _p, _p, ctypes.c_size_t, _p, _p]),
    "spec_verify_mixed_early_exit": (_i, [_p, _i, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p,
                                          ctypes.c_size_t, _p, _p]),
    "spec_draft_sample": (_i, [_p, _i, ctypes.c_int64, _p, _p, ctypes.c_float, _p, _i, _i, _i,
                               _p, _p, _p, _p, _p]),
    "spec_verify_sample_lq": (_i, [_p, _i, _p, ctypes.c_int64, _p, _p, _p, _p, ctypes.c_float,
                                   _i, _i, _i, _p, _p, _p, _p, ctypes.c_size_t, _p, _p]),
    "spec_verify_mixed_lq": (_i, [_p, _i, _p, ctypes.c_int64, _p, _p, _p, _p, _p,
                                  _i, _i, _i, _p, _p, _p, _p, ctypes.c_size_t, _p, _p]),
    "spec_verify_sample_lq_early_exit": (_i, [_p, _i, _p, ctypes.c_int64, _p, _p, _p, _p,
                                              ctypes.c_float, _i, _i, _i, _p, _p, _p, _p,
                                              ctypes.c_size_t, _p, _p]),
    "spec_verify_mixed_lq_early_exit": (_i, [_p, _i, _p, ctypes.c_int64, _p, _p, _p, _p, _p,
                                             _i, _i, _i, _p, _p, _p, _p, ctypes.c_size_t, _p,
                                             _p]),
    "spec_verify_tree": (_i, [_p, _i, _p, _p, _p, _p, ctypes.c_float, _i, _i, _i, _p, _p, _p, _p,
                              ctypes.c_size_t, _p, _p]),
    "spec_verify_tree_lq": (_i, [_p, _i, _p, ctypes.c_int64, _p, _p, _p, _p, _p, ctypes.c_float,
                                 _i, _i, _i, _p, _p, _p, _p, ctypes.c_size_t, _p, _p]),
    "spec_verify_tree_early_exit": (_i, [_p, _i, _p, _p, _p, _p, ctypes.c_float, _i, _i, _i, _p,
                                         _p, _p, _p, ctypes.c_size_t, _p, _p]),
    "spec_verify_tree_lq_early_exit": (_i, [_p, _i, _p, ctypes.c_int64, _p, _p, _p, _p, _p,
                                            ctypes.c_float, _i, _i, _i, _p, _p, _p, _p,
                                            ctypes.c_size_t, _p, _p]),
    "spec_verify_tree_mixed": (_i, [_p, _i, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p,
                                    ctypes.c_size_t, _p, _p]),
    "spec_verify_tree_mixed_early_exit": (_i, [_p, _i, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p,
                                               _p, _p, ctypes.c_size_t, _p, _p]),
    "spec_accept_metrics_words": (ctypes.c_size_t, [_i]),
    "spec_accept_metrics": (_i, [_p, _i, _i, _p, _p, _p]),
    "sv_step_graph_create": (_i, [_p, _p]),
    "sv_step_graph_launch": (_i, [_p, _p]),
    "sv_step_graph_destroy": (None, [_p]),
    "sv_kernel_name": (ctypes.c_char_p, [_i]),
    "sv_trace_begin": (_i, [_i, ctypes.c_uint]),
    "sv_trace_count": (_i, []),
    "sv_trace_read": (_i, [_i, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float)]),
    "sv_trace_end": (None, []),
    "sv_trace_enable": (None, [_i]),
}


class SpecVerifyError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def require_library():
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    lib = _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise SpecVerifyError(
                    f"{_LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
            lib = ctypes.CDLL(_LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def sv_status_string(status: int) -> str:
    return require_library().sv_status_string(status).decode()


_ws_bytes = {}


def spec_verify_workspace_bytes(B: int, K: int, V: int) -> int:
    key = (B, K, V)
    n = _ws_bytes.get(key)
    if n is None:
        n = _ws_bytes[key] = int(require_library().spec_verify_workspace_bytes(B, K, V))
    return n


def _check(status: int, what: str):
    if status != 0:
        raise SpecVerifyError(f"{what}: {sv_status_string(status)} (status {status})")


# ---------------------------------------------------------------- tracing
KERNEL_IDS = {"verify_greedy_rows": 0, "verify_sample_rows": 1, "verify_sample_draw": 2,
              "peagle_build": 3, "verify_greedy_accept": 4, "verify_sample_locate": 5,
              "draft_sample": 6, "verify_mixed_rows": 7, "accept_metrics": 8, "tree_rows": 9,
              "tree_walk": 10}


def trace_begin(capacity: int, kernels=None):
    """Start kernel tracing on this host thread for up to `capacity` launches
    of the named kernels (all kernels when `kernels` is None)."""
    mask = 0xFFFFFFFF if kernels is None else sum(1 << KERNEL_IDS[k] for k in kernels)
    _check(require_library().sv_trace_begin(int(capacity), mask), "sv_trace_begin")


def trace_read():
    """[(kernel name, duration ms)] of the launches traced so far (waits for them)."""
    lib = require_library()
    out = []
    kid, ms = ctypes.c_int(), ctypes.c_float()
    for i in range(lib.sv_trace_count()):
        _check(lib.sv_trace_read(i, ctypes.byref(kid), ctypes.byref(ms)), "sv_trace_read")
        out.append((lib.sv_kernel_name(kid.value).decode(), float(ms.value)))
    return out


def trace_end():
    require_library().sv_trace_end()


def trace_enable(on: bool):
    """Pause (False) or resume (True) the active trace of this host thread."""
    require_library().sv_trace_enable(1 if on else 0)


# ---------------------------------------------------------------- helpers
_DTYPES = {torch.float32: SV_F32, torch.bfloat16: SV_BF16, torch.float16: SV_F16}


# The checks below run on every call, so they use the cheapest tensor
# queries (a small verify call spends more time here than on the GPU).
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype is not dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device):
    """The current HIP stream of `device` (the library enqueues on it)."""
    if _raw_stream is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


_ws_cache = {}


def _workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-filled workspace per device.  The kernels leave it zero-filled,
    so it is reused without clearing; calls on one device must share a stream."""
    key = (device.type, device.index)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


# ---------------------------------------------------------------- verify
def spec_verify_greedy(target_logits: torch.Tensor, draft_tokens: torch.Tensor,
                       out_tokens: Optional[torch.Tensor] = None,
                       out_num_accepted: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None,
                       device_error: Optional[torch.Tensor] = None,
                       _symbol: str = "spec_verify_greedy"):
    """Greedy verify; see spec_verify_greedy in include/spec_verify.h.

    target_logits [B, K+1, V] float32/bfloat16, draft_tokens [B, K] int32.
    Returns (out_tokens [B, K+1] int32, num_accepted [B] int32).
    """
    lib = require_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    _dev(target_logits, "target_logits")
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if out_tokens is None \
        else _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev) if out_num_accepted is None \
        else _dev(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    need = spec_verify_workspace_bytes(B, K, V)
    if workspace is None:
        workspace = _workspace(dev, need)
    _dev(workspace, "workspace", device=dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    st = getattr(lib, _symbol)(_ptr(target_logits), _DTYPES[target_logits.dtype],
                               _ptr(draft_tokens), B, K, V, _ptr(out_tokens),
                               _ptr(out_num_accepted), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(device_error),
                               _stream(dev))
    _check(st, _symbol)
    return out_tokens, out_num_accepted


def spec_verify_sample(target_logits: torch.Tensor, draft_probs: torch.Tensor,
                       draft_tokens: torch.Tensor, uniforms: torch.Tensor, temperature: float,
                       out_tokens: Optional[torch.Tensor] = None,
                       out_num_accepted: Optional[torch.Tensor] = None,
                       out_draft_target_prob: Optional[torch.Tensor] = None,
                       want_draft_target_prob: bool = False,
                       workspace: Optional[torch.Tensor] = None,
                       device_error: Optional[torch.Tensor] = None,
                       _symbol: str = "spec_verify_sample"):
    """Rejection-sampling verify; see spec_verify_sample in include/spec_verify.h.

    Returns (out_tokens, num_accepted, draft_target_prob or None).
    """
    lib = require_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    _dev(target_logits, "target_logits")
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    _dev(draft_probs, "draft_probs", torch.float32, (B, K, V), dev)
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _dev(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if out_tokens is None \
        else _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev) if out_num_accepted is None \
        else _dev(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    if out_draft_target_prob is None and want_draft_target_prob:
        out_draft_target_prob = torch.empty((B, K), dtype=torch.float32, device=dev)
    if out_draft_target_prob is not None:
        _dev(out_draft_target_prob, "out_draft_target_prob", torch.float32, (B, K), dev)
    need = spec_verify_workspace_bytes(B, K, V)
    if workspace is None:
        workspace = _workspace(dev, need)
    _dev(workspace, "workspace", device=dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    st = getattr(lib, _symbol)(_ptr(target_logits), _DTYPES[target_logits.dtype], _ptr(draft_probs),
                                _ptr(draft_tokens), _ptr(uniforms), float(temperature), B, K, V,
                                _ptr(out_tokens), _ptr(out_num_accepted), _ptr(out_draft_target_prob),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _ptr(device_error), _stream(dev))
    _check(st, _symbol)
    return out_tokens, out_num_accepted, out_draft_target_prob


def noalloc_scratch_bytes() -> int:
    """Size of the fixed scratch array spec_verify_sample_noalloc uses per GPU."""
    return int(require_library().spec_verify_noalloc_scratch_bytes())


def spec_verify_sample_noalloc(target_logits: torch.Tensor, draft_probs: torch.Tensor,
                               draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                               temperature: float,
                               out_tokens: torch.Tensor, out_num_accepted: torch.Tensor,
                               out_draft_target_prob: Optional[torch.Tensor] = None,
                               device_error: Optional[torch.Tensor] = None):
    """spec_verify_sample without a workspace (see spec_verify_sample_noalloc in
    include/spec_verify.h): the library takes its scratch from a fixed device
    array, and the caller passes every output, so the call allocates nothing."""
    lib = require_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    _dev(target_logits, "target_logits")
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    _dev(draft_probs, "draft_probs", torch.float32, (B, K, V), dev)
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _dev(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    _dev(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    if out_draft_target_prob is not None:
        _dev(out_draft_target_prob, "out_draft_target_prob", torch.float32, (B, K), dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    st = lib.spec_verify_sample_noalloc(
        _ptr(target_logits), _DTYPES[target_logits.dtype], _ptr(draft_probs), _ptr(draft_tokens),
        _ptr(uniforms), float(temperature), B, K, V, _ptr(out_tokens), _ptr(out_num_accepted),
        _ptr(out_draft_target_prob), _ptr(device_error), _stream(dev))
    _check(st, "spec_verify_sample_noalloc")
    return out_tokens, out_num_accepted, out_draft_target_prob


def spec_verify_mixed(target_logits: torch.Tensor, draft_probs: torch.Tensor,
                      draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                      temperatures: torch.Tensor,
                      out_tokens: Optional[torch.Tensor] = None,
                      out_num_accepted: Optional[torch.Tensor] = None,
                      out_draft_target_prob: Optional[torch.Tensor] = None,
                      want_draft_target_prob: bool = False,
                      workspace: Optional[torch.Tensor] = None,
                      device_error: Optional[torch.Tensor] = None,
                      _symbol: str = "spec_verify_mixed"):
    """Verify with a temperature per sequence (0 = greedy); see
    spec_verify_mixed in include/spec_verify.h.

    Returns (out_tokens, num_accepted, draft_target_prob or None).
    """
    lib = require_library()
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, K+1, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    _dev(target_logits, "target_logits")
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    _dev(draft_probs, "draft_probs", torch.float32, (B, K, V), dev)
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _dev(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    _dev(temperatures, "temperatures", torch.float32, (B,), dev)
    out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if out_tokens is None \
        else _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev) if out_num_accepted is None \
        else _dev(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    if out_draft_target_prob is None and want_draft_target_prob:
        out_draft_target_prob = torch.empty((B, K), dtype=torch.float32, device=dev)
    if out_draft_target_prob is not None:
        _dev(out_draft_target_prob, "out_draft_target_prob", torch.float32, (B, K), dev)
    need = spec_verify_workspace_bytes(B, K, V)
    if workspace is None:
        workspace = _workspace(dev, need)
    _dev(workspace, "workspace", device=dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    st = getattr(lib, _symbol)(_ptr(target_logits), _DTYPES[target_logits.dtype],
                               _ptr(draft_probs), _ptr(draft_tokens), _ptr(uniforms),
                               _ptr(temperatures), B, K, V, _ptr(out_tokens),
                               _ptr(out_num_accepted), _ptr(out_draft_target_prob),
                               _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _ptr(device_error), _stream(dev))
    _check(st, _symbol)
    return out_tokens, out_num_accepted, out_draft_target_prob


def spec_verify_greedy_early_exit(*args, **kw):
    """spec_verify_greedy computing only the rows up to each sequence's first
    rejection; see spec_verify_greedy_early_exit in include/spec_verify.h.
    Arguments and results as spec_verify_greedy."""
    return spec_verify_greedy(*args, _symbol="spec_verify_greedy_early_exit", **kw)


def spec_verify_sample_early_exit(*args, **kw):
    """spec_verify_sample computing only the rows up to each sequence's first
    rejection; see spec_verify_sample_early_exit in include/spec_verify.h.
    Arguments as spec_verify_sample; draft_target_prob is 0 past num_accepted."""
    return spec_verify_sample(*args, _symbol="spec_verify_sample_early_exit", **kw)


def spec_verify_mixed_early_exit(*args, **kw):
    """spec_verify_mixed computing only the rows up to each sequence's first
    rejection; see spec_verify_mixed_early_exit in include/spec_verify.h.
    Arguments as spec_verify_mixed; draft_target_prob is 0 past num_accepted."""
    return spec_verify_mixed(*args, _symbol="spec_verify_mixed_early_exit", **kw)


# ---------------------------------------------------------------- P-EAGLE
def peagle_build_draft_batch(verify_out_tokens: torch.Tensor, num_accepted: torch.Tensor,
                             draft_tokens: torch.Tensor, start_pos: torch.Tensor,
                             block_table: torch.Tensor, block_size: int,
                             target_hidden: torch.Tensor, h_shared: torch.Tensor,
                             mask_token_id: int, outputs: Optional[dict] = None,
                             want_sample_rows: bool = True,
                             device_error: Optional[torch.Tensor] = None) -> dict:
    """P-EAGLE drafter batch; see peagle_build_draft_batch in include/spec_verify.h.

    Returns a dict of input_ids [B*2K] int32, positions [B*2K] int64,
    slot_mapping [B*2K] int64, hidden [B*2K, H], sample_rows [B, K] int32.
    """
    lib = require_library()
    B, K = draft_tokens.shape
    dev = draft_tokens.device
    H = target_hidden.shape[-1]
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _dev(verify_out_tokens, "verify_out_tokens", torch.int32, (B, K + 1), dev)
    _dev(num_accepted, "num_accepted", torch.int32, (B,), dev)
    _dev(start_pos, "start_pos", torch.int64, (B,), dev)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_blocks_per_seq]")
    _dev(block_table, "block_table", torch.int32, device=dev)
    if target_hidden.dtype not in _DTYPES:
        raise TypeError("hidden states must be bfloat16, float16 or float32")
    _dev(target_hidden, "target_hidden", shape=(B * (K + 1), H), device=dev)
    _dev(h_shared, "h_shared", target_hidden.dtype, (H,), dev)
    o = dict(outputs or {})
    n = B * 2 * K
    if "input_ids" not in o:
        o["input_ids"] = torch.empty(n, dtype=torch.int32, device=dev)
    if "positions" not in o:
        o["positions"] = torch.empty(n, dtype=torch.int64, device=dev)
    if "slot_mapping" not in o:
        o["slot_mapping"] = torch.empty(n, dtype=torch.int64, device=dev)
    if "hidden" not in o:
        o["hidden"] = torch.empty((n, H), dtype=target_hidden.dtype, device=dev)
    if "sample_rows" not in o and want_sample_rows:
        o["sample_rows"] = torch.empty((B, K), dtype=torch.int32, device=dev)
    _dev(o["input_ids"], "input_ids", torch.int32, (n,), dev)
    _dev(o["positions"], "positions", torch.int64, (n,), dev)
    _dev(o["slot_mapping"], "slot_mapping", torch.int64, (n,), dev)
    _dev(o["hidden"], "hidden", target_hidden.dtype, (n, H), dev)
    if o.get("sample_rows") is not None:
        _dev(o["sample_rows"], "sample_rows", torch.int32, (B, K), dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    st = lib.peagle_build_draft_batch(
        _ptr(verify_out_tokens), _ptr(num_accepted), _ptr(draft_tokens), _ptr(start_pos),
        _ptr(block_table), block_table.shape[1], int(block_size), _ptr(target_hidden), _ptr(h_shared),
        _DTYPES[target_hidden.dtype], int(mask_token_id), B, K, H, _ptr(o["input_ids"]),
        _ptr(o["positions"]), _ptr(o["slot_mapping"]), _ptr(o["hidden"]), _ptr(o.get("sample_rows")),
        _ptr(device_error), _stream(dev))
    _check(st, "peagle_build_draft_batch")
    return o


# ---------------------------------------------------------------- drafter outputs
def spec_draft_sample(drafter_logits: torch.Tensor, K: int, temperature: float,
                      uniforms: Optional[torch.Tensor] = None,
                      row_index: Optional[torch.Tensor] = None,
                      temperatures: Optional[torch.Tensor] = None,
                      out_draft_tokens: Optional[torch.Tensor] = None,
                      out_draft_probs: Optional[torch.Tensor] = None,
                      want_draft_probs: bool = True,
                      device_error: Optional[torch.Tensor] = None,
                      out_row_desc: Optional[torch.Tensor] = None,
                      want_row_desc: bool = False):
    """Sample the drafter's prediction rows; see spec_draft_sample in
    include/spec_verify.h.  drafter_logits is [n_rows, V]; B is taken from
    row_index ([B, K]) when given, else n_rows // K.

    Returns (draft_tokens [B, K] int32, draft_probs [B, K, V] fp32 or None),
    plus the row descriptors ([B, K, 4] int32 holding sv_draft_row) as a third
    element when want_row_desc or out_row_desc is given.
    """
    lib = require_library()
    if drafter_logits.dim() != 2:
        raise ValueError("drafter_logits must be [n_rows, V]")
    n_rows, V = drafter_logits.shape
    dev = drafter_logits.device
    _dev(drafter_logits, "drafter_logits")
    if drafter_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("drafter_logits must be float32 or bfloat16")
    if row_index is not None:
        if row_index.dim() != 2 or row_index.shape[1] != K:
            raise ValueError("row_index must be [B, K]")
        B = row_index.shape[0]
        _dev(row_index, "row_index", torch.int32, (B, K), dev)
    else:
        if K < 1 or n_rows % K:
            raise ValueError("without row_index, n_rows must be a multiple of K")
        B = n_rows // K
    if uniforms is not None:
        _dev(uniforms, "uniforms", torch.float32, (B, K), dev)
    if temperatures is not None:
        _dev(temperatures, "temperatures", torch.float32, (B,), dev)
    out_draft_tokens = torch.empty((B, K), dtype=torch.int32, device=dev) \
        if out_draft_tokens is None else _dev(out_draft_tokens, "out_draft_tokens", torch.int32,
                                             (B, K), dev)
    if out_draft_probs is None and want_draft_probs:
        out_draft_probs = torch.empty((B, K, V), dtype=torch.float32, device=dev)
    if out_draft_probs is not None:
        _dev(out_draft_probs, "out_draft_probs", torch.float32, (B, K, V), dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    with_desc = want_row_desc or out_row_desc is not None
    if out_row_desc is None and want_row_desc:
        out_row_desc = torch.empty((B, K, 4), dtype=torch.int32, device=dev)
    if out_row_desc is not None:
        _dev(out_row_desc, "out_row_desc", torch.int32, (B, K, 4), dev)
    st = lib.spec_draft_sample(_ptr(drafter_logits), _DTYPES[drafter_logits.dtype], n_rows,
                               _ptr(row_index), _ptr(uniforms), float(temperature),
                               _ptr(temperatures), B, K, V, _ptr(out_draft_tokens),
                               _ptr(out_draft_probs), _ptr(out_row_desc), _ptr(device_error),
                               _stream(dev))
    _check(st, "spec_draft_sample")
    if with_desc:
        return out_draft_tokens, out_draft_probs, out_row_desc
    return out_draft_tokens, out_draft_probs


def _verify_lq(name, target_logits, drafter_logits, drafter_desc, draft_tokens, uniforms,
               temperature, temperatures, drafter_rows, out_tokens, out_num_accepted,
               out_draft_target_prob, want_draft_target_prob, workspace, device_error):
    lib = require_library()
    if target_logits.dim() != 3 or drafter_logits.dim() != 2:
        raise ValueError("target_logits must be [B, K+1, V] and drafter_logits [n_rows, V]")
    B, K1, V = target_logits.shape
    K = K1 - 1
    dev = target_logits.device
    _dev(target_logits, "target_logits")
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    _dev(drafter_logits, "drafter_logits", target_logits.dtype, (drafter_logits.shape[0], V), dev)
    _dev(drafter_desc, "drafter_desc", torch.int32, (B, K, 4), dev)
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, K), dev)
    _dev(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    if temperatures is not None:
        _dev(temperatures, "temperatures", torch.float32, (B,), dev)
    if drafter_rows is not None:
        _dev(drafter_rows, "drafter_rows", torch.int32, (B, K), dev)
    out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev) if out_tokens is None \
        else _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1), dev)
    out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev) if out_num_accepted is None \
        else _dev(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    if out_draft_target_prob is None and want_draft_target_prob:
        out_draft_target_prob = torch.empty((B, K), dtype=torch.float32, device=dev)
    if out_draft_target_prob is not None:
        _dev(out_draft_target_prob, "out_draft_target_prob", torch.float32, (B, K), dev)
    need = spec_verify_workspace_bytes(B, K, V)
    if workspace is None:
        workspace = _workspace(dev, need)
    _dev(workspace, "workspace", device=dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    head = (_ptr(target_logits), _DTYPES[target_logits.dtype], _ptr(drafter_logits),
            drafter_logits.shape[0], _ptr(drafter_rows), _ptr(drafter_desc), _ptr(draft_tokens),
            _ptr(uniforms))
    tail = (B, K, V, _ptr(out_tokens), _ptr(out_num_accepted), _ptr(out_draft_target_prob),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(device_error),
            _stream(dev))
    if name.startswith("spec_verify_mixed_lq"):
        st = getattr(lib, name)(*head, _ptr(temperatures), *tail)
    else:
        st = getattr(lib, name)(*head, float(temperature), *tail)
    _check(st, name)
    return out_tokens, out_num_accepted, out_draft_target_prob


def spec_verify_sample_lq(target_logits: torch.Tensor, drafter_logits: torch.Tensor,
                          drafter_desc: torch.Tensor, draft_tokens: torch.Tensor,
                          uniforms: torch.Tensor, temperature: float,
                          drafter_rows: Optional[torch.Tensor] = None,
                          out_tokens: Optional[torch.Tensor] = None,
                          out_num_accepted: Optional[torch.Tensor] = None,
                          out_draft_target_prob: Optional[torch.Tensor] = None,
                          want_draft_target_prob: bool = False,
                          workspace: Optional[torch.Tensor] = None,
                          device_error: Optional[torch.Tensor] = None):
    """Sampled verify with q recomputed from the drafter logits and the row
    descriptors of spec_draft_sample; see spec_verify_sample_lq in
    include/spec_verify.h.  Returns (out_tokens, num_accepted, draft_target_prob
    or None)."""
    return _verify_lq("spec_verify_sample_lq", target_logits, drafter_logits, drafter_desc,
                      draft_tokens, uniforms, temperature, None, drafter_rows, out_tokens,
                      out_num_accepted, out_draft_target_prob, want_draft_target_prob,
                      workspace, device_error)


def spec_verify_mixed_lq(target_logits: torch.Tensor, drafter_logits: torch.Tensor,
                         drafter_desc: torch.Tensor, draft_tokens: torch.Tensor,
                         uniforms: torch.Tensor, temperatures: torch.Tensor,
                         drafter_rows: Optional[torch.Tensor] = None,
                         out_tokens: Optional[torch.Tensor] = None,
                         out_num_accepted: Optional[torch.Tensor] = None,
                         out_draft_target_prob: Optional[torch.Tensor] = None,
                         want_draft_target_prob: bool = False,
                         workspace: Optional[torch.Tensor] = None,
                         device_error: Optional[torch.Tensor] = None):
    """Mixed-batch verify (per-sequence temperatures, 0 = greedy) with q
    recomputed from the drafter logits and row descriptors; see
    spec_verify_mixed_lq in include/spec_verify.h.  Returns (out_tokens,
    num_accepted, draft_target_prob or None)."""
    return _verify_lq("spec_verify_mixed_lq", target_logits, drafter_logits, drafter_desc,
                      draft_tokens, uniforms, None, temperatures, drafter_rows, out_tokens,
                      out_num_accepted, out_draft_target_prob, want_draft_target_prob,
                      workspace, device_error)


def spec_verify_sample_lq_early_exit(target_logits, drafter_logits, drafter_desc, draft_tokens,
                                     uniforms, temperature, drafter_rows=None, out_tokens=None,
                                     out_num_accepted=None, out_draft_target_prob=None,
                                     want_draft_target_prob=False, workspace=None,
                                     device_error=None):
    """spec_verify_sample_lq computing only the rows up to each sequence's
    first rejection; see spec_verify_sample_lq_early_exit in
    include/spec_verify.h.  draft_target_prob is 0 past num_accepted."""
    return _verify_lq("spec_verify_sample_lq_early_exit", target_logits, drafter_logits,
                      drafter_desc, draft_tokens, uniforms, temperature, None, drafter_rows,
                      out_tokens, out_num_accepted, out_draft_target_prob,
                      want_draft_target_prob, workspace, device_error)


def spec_verify_mixed_lq_early_exit(target_logits, drafter_logits, drafter_desc, draft_tokens,
                                    uniforms, temperatures, drafter_rows=None, out_tokens=None,
                                    out_num_accepted=None, out_draft_target_prob=None,
                                    want_draft_target_prob=False, workspace=None,
                                    device_error=None):
    """spec_verify_mixed_lq computing only the rows up to each sequence's
    first rejection; see spec_verify_mixed_lq_early_exit in
    include/spec_verify.h.  draft_target_prob is 0 past num_accepted."""
    return _verify_lq("spec_verify_mixed_lq_early_exit", target_logits, drafter_logits,
                      drafter_desc, draft_tokens, uniforms, None, temperatures, drafter_rows,
                      out_tokens, out_num_accepted, out_draft_target_prob,
                      want_draft_target_prob, workspace, device_error)


# ---------------------------------------------------------------- draft trees
def spec_verify_tree(target_logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                     temperature: float = 0.0, draft_probs: Optional[torch.Tensor] = None,
                     uniforms: Optional[torch.Tensor] = None,
                     out_tokens: Optional[torch.Tensor] = None,
                     out_path: Optional[torch.Tensor] = None,
                     out_num_accepted: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     device_error: Optional[torch.Tensor] = None,
                     _symbol: str = "spec_verify_tree", _temperatures=None):
    """Verify a draft tree per sequence (temperature 0 = greedy); see
    spec_verify_tree in include/spec_verify.h.

    Returns (out_tokens [B, N+1], out_path [B, N+1], num_accepted [B])."""
    lib = require_library()
    mixed = _temperatures is not None
    if mixed:
        temperature = 1.0                  # per-tree temperatures instead
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B, N+1, V]")
    B, N1, V = target_logits.shape
    N = N1 - 1
    dev = target_logits.device
    _dev(target_logits, "target_logits")
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    _dev(parents, "parents", torch.int32, (B, N), dev)
    _dev(tokens, "tokens", torch.int32, (B, N), dev)
    if temperature > 0:
        _dev(draft_probs, "draft_probs", torch.float32, (B, N + 1, V), dev)
        _dev(uniforms, "uniforms", torch.float32, (B, N + 1), dev)
    out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev) if out_tokens is None \
        else _dev(out_tokens, "out_tokens", torch.int32, (B, N + 1), dev)
    out_path = torch.empty((B, N + 1), dtype=torch.int32, device=dev) if out_path is None \
        else _dev(out_path, "out_path", torch.int32, (B, N + 1), dev)
    out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev) if out_num_accepted is None \
        else _dev(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    need = spec_verify_workspace_bytes(B, N, V)
    if workspace is None:
        workspace = _workspace(dev, need)
    _dev(workspace, "workspace", device=dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    head = (_ptr(target_logits), _DTYPES[target_logits.dtype],
            _ptr(draft_probs if temperature > 0 else None), _ptr(parents), _ptr(tokens),
            _ptr(uniforms if temperature > 0 else None))
    tail = (B, N, V, _ptr(out_tokens), _ptr(out_path), _ptr(out_num_accepted), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(device_error), _stream(dev))
    if mixed:
        _dev(_temperatures, "temperatures", torch.float32, (B,), dev)
        st = getattr(lib, _symbol)(*head, _ptr(_temperatures), *tail)
    else:
        st = getattr(lib, _symbol)(*head, float(temperature), *tail)
    _check(st, _symbol)
    return out_tokens, out_path, out_num_accepted


def spec_verify_tree_mixed(target_logits, parents, tokens, temperatures, draft_probs, uniforms,
                           **kw):
    """Verify a mixed batch of draft trees (per-tree temperatures, 0 =
    greedy); see spec_verify_tree_mixed in include/spec_verify.h.  Keyword
    arguments and results as spec_verify_tree."""
    return spec_verify_tree(target_logits, parents, tokens, 1.0, draft_probs, uniforms,
                            _symbol="spec_verify_tree_mixed", _temperatures=temperatures, **kw)


def spec_verify_tree_mixed_early_exit(target_logits, parents, tokens, temperatures,
                                      draft_probs, uniforms, **kw):
    """spec_verify_tree_mixed with the walk computing the statistics of the
    rows it visits only; see spec_verify_tree_mixed_early_exit."""
    return spec_verify_tree(target_logits, parents, tokens, 1.0, draft_probs, uniforms,
                            _symbol="spec_verify_tree_mixed_early_exit",
                            _temperatures=temperatures, **kw)


def spec_verify_tree_lq(target_logits: torch.Tensor, drafter_logits: torch.Tensor,
                        drafter_desc: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor,
                        uniforms: torch.Tensor, temperature: float,
                        drafter_rows: Optional[torch.Tensor] = None,
                        out_tokens: Optional[torch.Tensor] = None,
                        out_path: Optional[torch.Tensor] = None,
                        out_num_accepted: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None,
                        device_error: Optional[torch.Tensor] = None,
                        _symbol: str = "spec_verify_tree_lq"):
    """Sampled tree verification with q recomputed from the drafter logits
    and the row descriptors of spec_draft_sample; see spec_verify_tree_lq in
    include/spec_verify.h.  drafter_desc is [B, N+1, 4] int32 (sv_draft_row),
    drafter_rows optional [B, N+1].

    Returns (out_tokens [B, N+1], out_path [B, N+1], num_accepted [B])."""
    lib = require_library()
    if target_logits.dim() != 3 or drafter_logits.dim() != 2:
        raise ValueError("target_logits must be [B, N+1, V] and drafter_logits [n_rows, V]")
    B, N1, V = target_logits.shape
    N = N1 - 1
    dev = target_logits.device
    _dev(target_logits, "target_logits")
    if target_logits.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("target_logits must be float32 or bfloat16")
    _dev(drafter_logits, "drafter_logits", target_logits.dtype, (drafter_logits.shape[0], V), dev)
    _dev(drafter_desc, "drafter_desc", torch.int32, (B, N + 1, 4), dev)
    _dev(parents, "parents", torch.int32, (B, N), dev)
    _dev(tokens, "tokens", torch.int32, (B, N), dev)
    _dev(uniforms, "uniforms", torch.float32, (B, N + 1), dev)
    if drafter_rows is not None:
        _dev(drafter_rows, "drafter_rows", torch.int32, (B, N + 1), dev)
    out_tokens = torch.empty((B, N + 1), dtype=torch.int32, device=dev) if out_tokens is None \
        else _dev(out_tokens, "out_tokens", torch.int32, (B, N + 1), dev)
    out_path = torch.empty((B, N + 1), dtype=torch.int32, device=dev) if out_path is None \
        else _dev(out_path, "out_path", torch.int32, (B, N + 1), dev)
    out_num_accepted = torch.empty(B, dtype=torch.int32, device=dev) if out_num_accepted is None \
        else _dev(out_num_accepted, "out_num_accepted", torch.int32, (B,), dev)
    need = spec_verify_workspace_bytes(B, N, V)
    if workspace is None:
        workspace = _workspace(dev, need)
    _dev(workspace, "workspace", device=dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    st = getattr(lib, _symbol)(_ptr(target_logits), _DTYPES[target_logits.dtype],
                                 _ptr(drafter_logits), drafter_logits.shape[0],
                                 _ptr(drafter_rows), _ptr(drafter_desc), _ptr(parents),
                                 _ptr(tokens), _ptr(uniforms), float(temperature), B, N, V,
                                 _ptr(out_tokens), _ptr(out_path), _ptr(out_num_accepted),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _ptr(device_error), _stream(dev))
    _check(st, _symbol)
    return out_tokens, out_path, out_num_accepted


def spec_verify_tree_early_exit(*args, **kw):
    """spec_verify_tree with the walk computing the statistics of the rows it
    visits only; see spec_verify_tree_early_exit in include/spec_verify.h.
    Arguments and results as spec_verify_tree."""
    return spec_verify_tree(*args, _symbol="spec_verify_tree_early_exit", **kw)


def spec_verify_tree_lq_early_exit(*args, **kw):
    """spec_verify_tree_lq with the walk computing the statistics of the rows
    it visits only; see spec_verify_tree_lq_early_exit in include/spec_verify.h."""
    return spec_verify_tree_lq(*args, _symbol="spec_verify_tree_lq_early_exit", **kw)


# ---------------------------------------------------------------- acceptance metrics
METRICS_STEPS, METRICS_ROUNDS, METRICS_PROPOSED, METRICS_ACCEPTED, METRICS_EMITTED, \
    METRICS_HIST = range(6)


def accept_metrics_buffer(K: int, device) -> torch.Tensor:
    """A zeroed counter array for spec_accept_metrics (int64 storage of the
    uint64 counters)."""
    n = require_library().spec_accept_metrics_words(int(K))
    if n == 0:
        raise ValueError(f"K={K} out of range")
    return torch.zeros(n, dtype=torch.int64, device=device)


def spec_accept_metrics(num_accepted: torch.Tensor, K: int, metrics: torch.Tensor,
                        device_error: Optional[torch.Tensor] = None):
    """Add one verify call's counts to `metrics`; see spec_accept_metrics in
    include/spec_verify.h."""
    lib = require_library()
    if num_accepted.dim() != 1:
        raise ValueError("num_accepted must be [B]")
    B = num_accepted.shape[0]
    dev = num_accepted.device
    _dev(num_accepted, "num_accepted", torch.int32, (B,), dev)
    _dev(metrics, "metrics", torch.int64, (lib.spec_accept_metrics_words(int(K)),), dev)
    if device_error is not None:
        _dev(device_error, "device_error", torch.int32, (1,), dev)
    _check(lib.spec_accept_metrics(_ptr(num_accepted), B, int(K), _ptr(metrics),
                                   _ptr(device_error), _stream(dev)), "spec_accept_metrics")
    return metrics


def acceptance_summary(metrics: torch.Tensor) -> dict:
    """Host-side view of the counters (synchronises): reads back the integer
    counters that spec_accept_metrics accumulated on the device and divides
    them into the acceptance length, tokens per round and draft acceptance
    rate.  A reporting convenience, not part of the path: every count is
    taken on the GPU, and the three ratios are plain quotients of them."""
    m = [int(x) for x in metrics.cpu().tolist()]
    rounds, proposed, accepted, emitted = (m[METRICS_ROUNDS], m[METRICS_PROPOSED],
                                           m[METRICS_ACCEPTED], m[METRICS_EMITTED])
    return {"steps": m[METRICS_STEPS], "rounds": rounds, "proposed": proposed,
            "accepted": accepted, "emitted": emitted, "hist": m[METRICS_HIST:],
            "acceptance_length": accepted / rounds if rounds else float("nan"),
            "tokens_per_round": emitted / rounds if rounds else float("nan"),
            "draft_acceptance_rate": accepted / proposed if proposed else float("nan")}


# ---------------------------------------------------------------- step graphs
STEP_GREEDY, STEP_SAMPLE, STEP_MIXED = 0, 1, 2


class _StepDesc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("target_logits", _p), ("logits_dtype", ctypes.c_int),
                ("draft_probs", _p), ("draft_tokens", _p), ("uniforms", _p),
                ("temperature", ctypes.c_float), ("temperatures", _p),
                ("B", ctypes.c_int), ("K", ctypes.c_int), ("V", ctypes.c_int),
                ("out_tokens", _p), ("out_num_accepted", _p), ("out_draft_target_prob", _p),
                ("workspace", _p), ("workspace_bytes", ctypes.c_size_t),
                ("start_pos", _p), ("block_table", _p), ("max_blocks_per_seq", ctypes.c_int),
                ("block_size", ctypes.c_int), ("target_hidden", _p), ("h_shared", _p),
                ("hidden_dtype", ctypes.c_int), ("mask_token_id", ctypes.c_int32),
                ("H", ctypes.c_int), ("out_input_ids", _p), ("out_positions", _p),
                ("out_slot_mapping", _p), ("out_hidden", _p), ("out_sample_rows", _p),
                ("metrics", _p), ("device_error", _p),
                ("drafter_logits", _p), ("n_drafter_rows", ctypes.c_int64),
                ("drafter_rows", _p), ("drafter_desc", _p), ("early_exit", ctypes.c_int)]


class StepGraph:
    """One decode step (verify, then optionally the P-EAGLE build and the
    acceptance metrics) captured as a HIP graph; see sv_step_graph_create in
    include/spec_verify.h.  Every tensor is fixed at capture and kept alive
    by this object; ``launch()`` replays the step on the current stream with
    whatever the tensors hold.

    verify: dict with target_logits, draft_tokens, out_tokens,
      out_num_accepted, workspace, and for sampling draft_probs, uniforms and
      temperature (mode "sample") or temperatures (mode "mixed"); optional
      out_draft_target_prob.  For sampling with q from the drafter logits,
      drafter_logits ([n_rows, V]) and drafter_desc ([B, K, 4] int32, from
      spec_draft_sample) replace draft_probs, with an optional drafter_rows
      ([B, K] int32).
    build: None, or dict with start_pos, block_table, block_size,
      target_hidden, h_shared, mask_token_id and outputs (as returned by
      peagle_build_draft_batch or preallocated).
    metrics: None, or a counter array from accept_metrics_buffer.
    early_exit: capture the _early_exit form of the verify.
    """

    def __init__(self, mode: str, verify: dict, build: Optional[dict] = None,
                 metrics: Optional[torch.Tensor] = None,
                 device_error: Optional[torch.Tensor] = None, early_exit: bool = False):
        lib = require_library()
        z = verify["target_logits"]
        if z.dim() != 3:
            raise ValueError("target_logits must be [B, K+1, V]")
        B, K1, V = z.shape
        K = K1 - 1
        dev = z.device
        d = _StepDesc()
        d.mode = {"greedy": STEP_GREEDY, "sample": STEP_SAMPLE, "mixed": STEP_MIXED}[mode]
        d.early_exit = 1 if early_exit else 0
        keep = [z]

        def ptr(t, name, dtype=None, shape=None):
            if t is None:
                return None
            _dev(t, name, dtype, shape, dev)
            keep.append(t)
            return t.data_ptr()

        d.target_logits = ptr(z, "target_logits")
        d.logits_dtype = _DTYPES[z.dtype]
        d.draft_tokens = ptr(verify["draft_tokens"], "draft_tokens", torch.int32, (B, K))
        zd = verify.get("drafter_logits")
        if zd is not None:
            if mode == "greedy" or verify.get("draft_probs") is not None:
                raise ValueError("drafter_logits replaces draft_probs, for sampling only")
            if zd.dim() != 2 or zd.shape[1] != V or zd.dtype != z.dtype:
                raise ValueError("drafter_logits must be [n_rows, V] in the target's dtype")
            d.drafter_logits = ptr(zd, "drafter_logits")
            d.n_drafter_rows = zd.shape[0]
            d.drafter_rows = ptr(verify.get("drafter_rows"), "drafter_rows", torch.int32, (B, K))
            d.drafter_desc = ptr(verify["drafter_desc"], "drafter_desc", torch.int32, (B, K, 4))
        if mode != "greedy":
            if zd is None:
                d.draft_probs = ptr(verify["draft_probs"], "draft_probs", torch.float32,
                                    (B, K, V))
            d.uniforms = ptr(verify["uniforms"], "uniforms", torch.float32, (B, K + 1))
        if mode == "sample":
            d.temperature = float(verify["temperature"])
        if mode == "mixed":
            d.temperatures = ptr(verify["temperatures"], "temperatures", torch.float32, (B,))
        d.B, d.K, d.V = B, K, V
        d.out_tokens = ptr(verify["out_tokens"], "out_tokens", torch.int32, (B, K + 1))
        d.out_num_accepted = ptr(verify["out_num_accepted"], "out_num_accepted", torch.int32, (B,))
        d.out_draft_target_prob = ptr(verify.get("out_draft_target_prob"), "out_draft_target_prob",
                                      torch.float32, (B, K))
        ws = verify["workspace"]
        d.workspace = ptr(ws, "workspace")
        d.workspace_bytes = ws.numel() * ws.element_size()
        if build is not None:
            h = build["target_hidden"]
            H = h.shape[1]
            o = build["outputs"]
            d.start_pos = ptr(build["start_pos"], "start_pos", torch.int64, (B,))
            bt = build["block_table"]
            d.block_table = ptr(bt, "block_table", torch.int32)
            d.max_blocks_per_seq = bt.shape[1]
            d.block_size = int(build["block_size"])
            d.target_hidden = ptr(h, "target_hidden", None, (B * (K + 1), H))
            d.h_shared = ptr(build["h_shared"], "h_shared", h.dtype, (H,))
            d.hidden_dtype = _DTYPES[h.dtype]
            d.mask_token_id = int(build["mask_token_id"])
            d.H = H
            d.out_input_ids = ptr(o["input_ids"], "input_ids", torch.int32, (B * 2 * K,))
            d.out_positions = ptr(o["positions"], "positions", torch.int64, (B * 2 * K,))
            d.out_slot_mapping = ptr(o["slot_mapping"], "slot_mapping", torch.int64, (B * 2 * K,))
            d.out_hidden = ptr(o["hidden"], "hidden", h.dtype, (B * 2 * K, H))
            d.out_sample_rows = ptr(o.get("sample_rows"), "sample_rows", torch.int32, (B, K))
        if metrics is not None:
            d.metrics = ptr(metrics, "metrics", torch.int64)
        if device_error is not None:
            d.device_error = ptr(device_error, "device_error", torch.int32, (1,))
        self._keep = keep
        self._desc = d
        self._lib = lib
        self._dev = dev
        self._g = ctypes.c_void_p()
        _check(lib.sv_step_graph_create(ctypes.byref(d), ctypes.byref(self._g)),
               "sv_step_graph_create")

    def launch(self):
        _check(self._lib.sv_step_graph_launch(self._g, _stream(self._dev)), "sv_step_graph_launch")

    def close(self):
        if self._g:
            self._lib.sv_step_graph_destroy(self._g)
            self._g = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
