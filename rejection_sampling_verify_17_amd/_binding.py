"""ctypes binding of libspecverify.so: argument marshalling only.

Every step of the verification runs in the library's HIP kernels; this module
checks tensors, allocates outputs and a workspace with torch, and
passes raw device pointers plus the current HIP stream.  If the library is
missing it raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SV_F32 = 0
SV_BF16 = 1
SV_OK = 0
SV_EINVAL = 1
SV_EHIP = 2
NOALLOC_WORKSPACE_BYTES = 32 << 20   # SV_NOALLOC_WORKSPACE_BYTES of include/specverify.h


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = ""
        if status == SV_EHIP:
            self.hip_error = int(lib().sv_last_hip_error())
            detail = f", hipError_t {self.hip_error}"
        super().__init__(f"{where}: {status_string(status)} (status {status}{detail})")


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise ImportError(
                        f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
                # torch ships its own HIP runtime under the same soname as the
                # system's; loading this library first would make torch bind to
                # the system copy, and launches then fail (hipErrorNoDevice).
                # Importing torch first keeps one runtime in the process: torch's.
                try:
                    import torch  # noqa: F401
                except ImportError:
                    pass
                L = ctypes.CDLL(LIB_PATH)
                vp, i32, u64, flt, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float,
                                         ctypes.c_size_t)
                common = [vp, vp, vp, i32, i32, i32, i32, flt, i32, flt, u64, u64, vp, vp, vp, sz, vp]
                L.sv_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
                L.sv_workspace_bytes.restype = sz
                L.sv_verify.argtypes = common
                L.sv_verify.restype = i32
                L.sv_verify_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, i32, flt, i32, flt, u64, u64, vp, vp, vp]
                L.sv_verify_noalloc.restype = i32
                L.sv_verify_debug.argtypes = common + [vp, vp]
                L.sv_verify_debug.restype = i32
                L.sv_verify_timed.argtypes = common + [vp, i32, vp]
                L.sv_verify_timed.restype = i32
                L.sv_launch_name.argtypes = [i32, i32, i32, i32, i32, flt, flt, i32]
                L.sv_launch_name.restype = ctypes.c_char_p
                L.sv_draft_sample.argtypes = [vp, i32, i32, i32, i32, flt, i32, flt, u64, u64, vp, vp]
                L.sv_draft_sample.restype = i32
                L.sv_accept_histogram.argtypes = [vp, i32, i32, vp, vp]
                L.sv_accept_histogram.restype = i32
                L.sv_probe_read.argtypes = [vp, sz, vp, i32, i32, vp]
                L.sv_probe_read.restype = i32
                L.sv_probe_variates.argtypes = [ctypes.c_uint32, i32, vp, vp]
                L.sv_probe_variates.restype = i32
                L.sv_probe_math.argtypes = [vp, i32, i32, vp, vp]
                L.sv_probe_math.restype = i32
                L.sv_last_hip_error.argtypes = []
                L.sv_last_hip_error.restype = i32
                L.sv_status_string.argtypes = [i32]
                L.sv_status_string.restype = ctypes.c_char_p
                L.sv_version.argtypes = []
                L.sv_version.restype = ctypes.c_char_p
                _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().sv_status_string(s).decode()


def version() -> str:
    return lib().sv_version().decode()


def workspace_bytes(B: int, gamma: int, V: int, top_k: int, dtype: int) -> int:
    return int(lib().sv_workspace_bytes(B, gamma, V, top_k, dtype))


def launch_names(B: int, gamma: int, V: int, dtype: int, top_k: int, temperature: float = 1.0,
                 top_p: float = 1.0) -> list[str]:
    out, i = [], 0
    while True:
        n = lib().sv_launch_name(B, gamma, V, dtype, top_k, float(top_p), float(temperature), i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


# ---------------------------------------------------------------------------
# torch front end
# ---------------------------------------------------------------------------
_workspaces: dict = {}


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _stream_ptr(device, stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return int(s.cuda_stream)


def get_workspace(device, nbytes: int, stream=None):
    """A workspace of at least nbytes for (device, stream), reused across calls
    (its contents between calls do not matter)."""
    torch = _torch()
    key = (device.index, _stream_ptr(device, stream))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream) if stream is not None else _nullctx():
            ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def _check(target, draft, tokens):
    torch = _torch()
    if not (target.is_cuda and draft.is_cuda and tokens.is_cuda):
        raise ValueError("target, draft and tokens must be GPU tensors")
    if not (target.device == draft.device == tokens.device):
        raise ValueError("target, draft and tokens must be on the same device")
    if target.dim() != 3 or draft.dim() != 3 or tokens.dim() != 2:
        raise ValueError("expected target [B, gamma+1, V], draft [B, gamma, V], tokens [B, gamma]")
    B, g1, V = target.shape
    if tuple(draft.shape) != (B, g1 - 1, V) or tuple(tokens.shape) != (B, g1 - 1):
        raise ValueError(f"shape mismatch: target {tuple(target.shape)}, draft {tuple(draft.shape)}, "
                         f"tokens {tuple(tokens.shape)}")
    if target.dtype != draft.dtype:
        raise TypeError("target and draft logits must share a dtype")
    if not (target.is_contiguous() and draft.is_contiguous()):
        raise ValueError("logits must be contiguous")
    if tokens.dtype == torch.int64:
        tokens = tokens.to(torch.int32)
    if tokens.dtype != torch.int32:
        raise TypeError("draft tokens must be int32 (or int64, converted)")
    return tokens.contiguous(), B, g1 - 1, V


def _run(fn_name, target, draft, tokens, temperature, top_k, seed, seq_offset, out_tokens, n_accepted,
         workspace, stream, extra, top_p=1.0):
    torch = _torch()
    tokens, B, gamma, V = _check(target, draft, tokens)
    dt = _dtype_code(target)
    dev = target.device
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    need = workspace_bytes(B, gamma, V, top_k, dt)
    if need == 0:
        raise SpecVerifyError(SV_EINVAL, "sv_workspace_bytes")
    ws = workspace if workspace is not None else get_workspace(dev, need, stream)
    with torch.cuda.device(dev):
        st = getattr(lib(), fn_name)(
            target.data_ptr(), draft.data_ptr(), tokens.data_ptr(), B, gamma, V, dt, float(temperature),
            int(top_k), float(top_p), int(seed) & 0xFFFFFFFFFFFFFFFF, int(seq_offset) & 0xFFFFFFFFFFFFFFFF,
            out_tokens.data_ptr(), n_accepted.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(dev, stream),
            *extra)
    if st != SV_OK:
        raise SpecVerifyError(st, fn_name)
    return out_tokens, n_accepted


def verify(target, draft, tokens, temperature: float, top_k: int = 0, seed: int = 0, seq_offset: int = 0,
           out_tokens=None, n_accepted=None, workspace=None, stream=None, top_p: float = 1.0):
    """One verification step (sv_verify).  target [B, gamma+1, V], draft
    [B, gamma, V] (float32 or bfloat16, contiguous, on the GPU), tokens
    [B, gamma] int32.  Returns (out_tokens [B, gamma+1], n_accepted [B]),
    enqueued on the current stream (no synchronisation)."""
    return _run("sv_verify", target, draft, tokens, temperature, top_k, seed, seq_offset, out_tokens,
                n_accepted, workspace, stream, (), top_p)


def verify_noalloc(target, draft, tokens, temperature: float, top_k: int = 0, seed: int = 0, seq_offset: int = 0,
                   out_tokens=None, n_accepted=None, stream=None, top_p: float = 1.0):
    """sv_verify_noalloc: sv_verify on the library's own fixed workspace (no
    workspace argument; the library allocates nothing).  Pass out_tokens
    [B, gamma+1] and n_accepted [B] (int32, on the logits' device) to allocate
    nothing here either.  Calls that overlap on one GPU race (one buffer per
    GPU)."""
    torch = _torch()
    tokens, B, gamma, V = _check(target, draft, tokens)
    dev = target.device
    if out_tokens is None:
        out_tokens = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    if n_accepted is None:
        n_accepted = torch.empty((B,), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        st = lib().sv_verify_noalloc(
            target.data_ptr(), draft.data_ptr(), tokens.data_ptr(), B, gamma, V, _dtype_code(target),
            float(temperature), int(top_k), float(top_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
            int(seq_offset) & 0xFFFFFFFFFFFFFFFF, out_tokens.data_ptr(), n_accepted.data_ptr(),
            _stream_ptr(dev, stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_verify_noalloc")
    return out_tokens, n_accepted


def verify_debug(target, draft, tokens, temperature: float, top_k: int = 0, seed: int = 0,
                 seq_offset: int = 0, workspace=None, stream=None, top_p: float = 1.0):
    """sv_verify_debug: also returns token_probs [B, gamma, 2] (p(t), q(t)) and
    accept_ur [B, gamma, 2] (u, ratio) as float32 tensors."""
    torch = _torch()
    B, g1, V = target.shape
    tp = torch.empty((B, g1 - 1, 2), dtype=torch.float32, device=target.device)
    ur = torch.empty((B, g1 - 1, 2), dtype=torch.float32, device=target.device)
    out, n = _run("sv_verify_debug", target, draft, tokens, temperature, top_k, seed, seq_offset, None, None,
                  workspace, stream, (tp.data_ptr(), ur.data_ptr()), top_p)
    return out, n, tp, ur


def verify_timed(target, draft, tokens, temperature: float, events, top_k: int = 0, seed: int = 0,
                 seq_offset: int = 0, out_tokens=None, n_accepted=None, workspace=None, stream=None,
                 top_p: float = 1.0):
    """sv_verify_timed: `events` is a sequence of hipEvent_t handles (ints),
    recorded before/after each launch.  Returns (out, n, number of launches)."""
    arr = (ctypes.c_void_p * len(events))(*events)
    nl = ctypes.c_int32(0)
    out, n = _run("sv_verify_timed", target, draft, tokens, temperature, top_k, seed, seq_offset, out_tokens,
                  n_accepted, workspace, stream, (ctypes.cast(arr, ctypes.c_void_p), len(events),
                                                  ctypes.addressof(nl)), top_p)
    return out, n, nl.value


def draft_sample(draft, temperature: float, top_k: int = 0, seed: int = 0, seq_offset: int = 0, out=None,
                 stream=None, top_p: float = 1.0):
    """sv_draft_sample: draft tokens [B, gamma] int32 drawn on the GPU from the
    draft rows [B, gamma, V] (float32 or bfloat16, contiguous)."""
    torch = _torch()
    if not draft.is_cuda or draft.dim() != 3 or not draft.is_contiguous():
        raise ValueError("draft must be a contiguous [B, gamma, V] GPU tensor")
    B, gamma, V = draft.shape
    dt = _dtype_code(draft)
    dev = draft.device
    if out is None:
        out = torch.empty((B, gamma), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        st = lib().sv_draft_sample(draft.data_ptr(), B, gamma, V, dt, float(temperature), int(top_k), float(top_p),
                                   int(seed) & 0xFFFFFFFFFFFFFFFF, int(seq_offset) & 0xFFFFFFFFFFFFFFFF,
                                   out.data_ptr(), _stream_ptr(dev, stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_draft_sample")
    return out


def accept_histogram(n_accepted, gamma: int, out=None, stream=None):
    """sv_accept_histogram: int32 [gamma + 2] counts (invalid, then n = 0..gamma)."""
    torch = _torch()
    if not n_accepted.is_cuda or n_accepted.dtype != torch.int32 or n_accepted.dim() != 1:
        raise ValueError("n_accepted must be a 1-D int32 GPU tensor")
    dev = n_accepted.device
    if out is None:
        out = torch.empty((gamma + 2,), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        st = lib().sv_accept_histogram(n_accepted.contiguous().data_ptr(), n_accepted.shape[0], int(gamma),
                                       out.data_ptr(), _stream_ptr(dev, stream))
    if st != SV_OK:
        raise SpecVerifyError(st, "sv_accept_histogram")
    return out
