"""MI355X MoE token dispatch / reduce-once combine / fused residual + RMSNorm.

Thin Python binding over the C ABI of ``libmoe_a2a.so`` (declared in
``include/moe_a2a.h``).  Every step of the path runs in the library's gfx950
kernels; this module only checks tensor shapes and dtypes, passes raw device
pointers and the current HIP stream, and turns return codes into exceptions.
PyTorch provides device memory and streams.  There is no fallback: if the
library is missing the import of the functions fails loudly.

The per-call functions go through ``_moe_fast``, a small CPython extension
linked to the same library that converts the arguments in C (ctypes costs
more per call than a decode-sized launch); the rest use ctypes.

Functions carry the C names:

  moe_dispatch, moe_dispatch_fp8, moe_combine, moe_combine_residual_rmsnorm, moe_route_counts,
  moe_sync_status, moe_reset, moe_output_is_reduced, moe_strerror,
  moe_workspace_bytes, moe_scratch_bytes, moe_last_hip_error,
  moe_partials_reduce, moe_partials_reduce_residual_rmsnorm

and ``MoeA2A`` owns one ``moe_handle`` plus the device buffers it binds (the
two partials functions take no handle).
"""
from __future__ import annotations

import ctypes
import importlib
import os
import sysconfig
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libmoe_a2a.so")
FAST_MODULE = os.path.join(PKG, "_moe_fast" + sysconfig.get_config_var("EXT_SUFFIX"))

MOE_OK = 0
MOE_ERR_ARG = -1
MOE_ERR_PHASE = -2
MOE_ERR_OVERFLOW = -3
MOE_ERR_EXPERT_ID = -4
MOE_ERR_HIP = -5
MOE_ERR_NOALLOC_SIZE = -6
MOE_ERR_GAVE_UP = -7
MOE_NOALLOC_MAX_ITEMS = 1048576
MOE_LAYOUT_PER_COPY = 0
MOE_LAYOUT_PER_REGION = 1
LAYOUTS = {"copy": MOE_LAYOUT_PER_COPY, "region": MOE_LAYOUT_PER_REGION}
MOE_STATUS_OVERFLOW = 1
MOE_STATUS_EXPERT_ID = 2
MOE_STATUS_GAVE_UP = 4
MOE_MAX_EP = 256
MOE_MAX_TOP_K = 64
MOE_MAX_FUSED_HIDDEN = 16384
MOE_MAX_HIDDEN = 1048576
MOE_MAX_TOKENS = 8388608
MOE_MAX_PARTIALS = 64

EXPORTED = (
    "moe_workspace_bytes", "moe_scratch_bytes", "moe_init", "moe_dispatch", "moe_dispatch_fp8",
    "moe_combine",
    "moe_combine_residual_rmsnorm", "moe_route_counts", "moe_sync_status", "moe_reset",
    "moe_output_is_reduced", "moe_strerror", "moe_partials_reduce",
    "moe_partials_reduce_residual_rmsnorm", "moe_last_hip_error", "moe_dispatch_noalloc",
)


class MoeHandle(ctypes.Structure):
    """Mirror of ``struct moe_handle``."""
    _fields_ = [
        ("max_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("ep_size", ctypes.c_int32), ("experts_per_rank", ctypes.c_int32),
        ("max_tokens_per_rank", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("counts", ctypes.c_void_p), ("src_index", ctypes.c_void_p),
        ("slot_index", ctypes.c_void_p), ("status", ctypes.c_void_p),
        ("scratch", ctypes.c_void_p), ("scratch_bytes", ctypes.c_size_t),
        ("phase", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
        ("runtime_max_tokens_per_rank", ctypes.c_int32), ("hip_error", ctypes.c_int32),
        ("onepass_epoch", ctypes.c_uint32), ("onepass_spin_limit", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {moe_strerror(code)} (code {code})" if what else moe_strerror(code))


_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it with "
                               "`python -m combine_moe_dispatch_03_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        H = ctypes.POINTER(MoeHandle)
        sig = {
            "moe_workspace_bytes": (SZ, [I32, I32, I32]),
            "moe_scratch_bytes": (SZ, [I32, I32, I32]),
            "moe_init": (ctypes.c_int, [H, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, SZ]),
            "moe_dispatch": (ctypes.c_int, [H, P, P, I32, I32, P, P]),
            "moe_dispatch_fp8": (ctypes.c_int, [H, P, P, I32, I32, P, P, P]),
            "moe_dispatch_noalloc": (ctypes.c_int, [H, P, P, I32, I32, P, P]),
            "moe_combine": (ctypes.c_int, [H, P, P, I32, P, P]),
            "moe_combine_residual_rmsnorm": (ctypes.c_int,
                                             [H, P, P, I32, P, P, P, ctypes.c_float, P, P]),
            "moe_route_counts": (ctypes.c_int, [H, P, I32, P]),
            "moe_sync_status": (ctypes.c_int, [H, P, ctypes.POINTER(I32)]),
            "moe_reset": (ctypes.c_int, [H]),
            "moe_output_is_reduced": (ctypes.c_int, []),
            "moe_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "moe_last_hip_error": (ctypes.c_int, []),
            "moe_partials_reduce": (ctypes.c_int, [P, I32, I32, I32, P, P]),
            "moe_partials_reduce_residual_rmsnorm": (
                ctypes.c_int, [P, I32, I32, I32, P, P, P, ctypes.c_float, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


_fast_mod = None


def _fast():
    """The ``_moe_fast`` extension: the per-call entry points (dispatch,
    dispatch_fp8, combine, combine_residual_rmsnorm, route_counts and the two
    partials reductions) with their argument conversion in C, a few
    microseconds cheaper per call than ctypes.  It calls the same functions
    of the same loaded library."""
    global _fast_mod
    if _fast_mod is None:
        library()                       # the library first: one copy, loaded by path
        if not os.path.exists(FAST_MODULE):
            raise RuntimeError(f"{FAST_MODULE} is missing: build it with "
                               "`python -m combine_moe_dispatch_03_amd.build`")
        _fast_mod = importlib.import_module(__name__ + "._moe_fast")
    return _fast_mod


# ---------------------------------------------------------------- helpers

def _current_stream_slow(device_index: int) -> int:
    return torch.cuda.current_stream(device_index).cuda_stream


# The current stream's raw handle without building a torch Stream object
# (that costs a few microseconds per call and would dominate a decode step).
# The fast query is torch-internal; if a torch version lacks it, the public
# (slower) one is used.
_current_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", _current_stream_slow)


def _stream(stream, device_index: int) -> int:
    """Raw HIP stream handle: the given stream, else the current stream of the
    handle's device."""
    if stream is None:
        return _current_raw_stream(device_index)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dev: int, shape=None, numel=None):
    # One combined test on the common path (get_device() is -1 off the GPU);
    # the messages are built only on failure.  Each tensor attribute read
    # costs ~0.1 us, and a decode step checks six tensors.
    try:
        if (t.dtype is dtype and t.get_device() == dev and t.is_contiguous()
                and (shape is None or t.shape == shape) and (numel is None or t.numel() == numel)):
            return
    except AttributeError:
        pass
    _need_failed(t, name, dtype, dev, shape, numel)


def _need_failed(t, name, dtype, dev, shape, numel):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.get_device() != dev:
        raise ValueError(f"{name} must be on the handle's device cuda:{dev}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _check(code: int, what: str) -> None:
    if code != MOE_OK:
        raise MoeError(code, what)


# ---------------------------------------------------------------- C names

def moe_workspace_bytes(ep_size: int, max_tokens_per_rank: int, hidden: int) -> int:
    return library().moe_workspace_bytes(ep_size, max_tokens_per_rank, hidden)


def moe_scratch_bytes(max_tokens: int, top_k: int, ep_size: int) -> int:
    return library().moe_scratch_bytes(max_tokens, top_k, ep_size)


def moe_output_is_reduced() -> bool:
    return bool(library().moe_output_is_reduced())


def moe_strerror(code: int) -> str:
    return library().moe_strerror(code).decode()


def moe_last_hip_error() -> int:
    """hipError_t behind this thread's most recent MOE_ERR_HIP (0 if none)."""
    return library().moe_last_hip_error()


class MoeA2A:
    """One ``moe_handle`` and the device buffers it binds (allocated once at
    the ladder maximum).  ``layout`` is "copy" (one workspace row per routed
    copy) or "region" (one row per token and destination region)."""

    def __init__(self, max_tokens: int, hidden: int, top_k: int, num_experts: int,
                 ep_size: int, max_tokens_per_rank: int, device=None, layout: str = "copy",
                 scratch: bool = True):
        dev = torch.device(device if device is not None else "cuda")
        if dev.type != "cuda":          # the handle's index buffers are written by kernels
            raise ValueError(f"MoeA2A needs a GPU device, got {dev}")
        lib = library()
        self.handle = MoeHandle()
        nbytes = lib.moe_scratch_bytes(max_tokens, top_k, ep_size)
        if nbytes == 0:
            raise MoeError(MOE_ERR_ARG, "moe_scratch_bytes")
        i32 = dict(dtype=torch.int32, device=dev)
        self.counts = torch.zeros(ep_size, **i32)
        self.src_index = torch.full((ep_size * max_tokens_per_rank,), -1, **i32)
        self.slot_index = torch.full((max_tokens * top_k,), -1, **i32)
        self.status = torch.zeros(1, **i32)
        # scratch=False binds none: the handle then serves moe_dispatch_noalloc only
        self.scratch = torch.zeros((nbytes + 3) // 4, **i32) if scratch else None
        if layout not in LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
        _check(lib.moe_init(ctypes.byref(self.handle), max_tokens, hidden, top_k, num_experts,
                            ep_size, max_tokens_per_rank, LAYOUTS[layout],
                            _ptr(self.counts), _ptr(self.src_index),
                            _ptr(self.slot_index), _ptr(self.status), _ptr(self.scratch),
                            self.scratch.numel() * 4 if scratch else 0), "moe_init")
        self.device = dev
        self.device_index = dev.index if dev.index is not None else torch.cuda.current_device()
        self.ref = ctypes.byref(self.handle)     # built once, passed on ctypes calls
        self.addr = ctypes.addressof(self.handle)  # passed to the _moe_fast calls
        # Sizes fixed by moe_init, kept as plain ints: the per-call checks read
        # them, and a ctypes field read costs several times an attribute read.
        self.hidden = hidden
        self.top_k = top_k
        self.ep_size = ep_size
        self.cap = max_tokens_per_rank
        self.workspace_numel = ep_size * max_tokens_per_rank * hidden
        self.layout = layout

    @property
    def num_tokens(self) -> int: return self.handle.num_tokens

    def new_workspace(self, fill_bits: Optional[int] = None) -> torch.Tensor:
        """A [ep, cap, H] bf16 workspace; optionally every element set to one
        bf16 bit pattern (e.g. a NaN canary for the padding)."""
        shape = (self.ep_size, self.cap, self.hidden)
        if fill_bits is None:
            return torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        w = torch.empty(shape, dtype=torch.int16, device=self.device)
        w.fill_(fill_bits - 65536 if fill_bits >= 32768 else fill_bits)
        return w.view(torch.bfloat16)

    def new_workspace_fp8(self, fill_byte: Optional[int] = None) -> torch.Tensor:
        """A [ep, cap, H] uint8 workspace for e4m3 codes (optionally filled)."""
        w = torch.empty((self.ep_size, self.cap, self.hidden), dtype=torch.uint8, device=self.device)
        if fill_byte is not None:
            w.fill_(fill_byte)
        return w

    def new_scales(self) -> torch.Tensor:
        """A [ep, cap] fp32 buffer for the fp8 row scales (filled with NaN)."""
        return torch.full((self.ep_size, self.cap), float("nan"), dtype=torch.float32,
                          device=self.device)

    def slot_index_view(self) -> torch.Tensor:
        T, k = self.handle.num_tokens, self.top_k
        return self.slot_index[: T * k].view(T, k)

    def src_index_view(self) -> torch.Tensor:
        return self.src_index.view(self.ep_size, self.cap)


def moe_dispatch(h: MoeA2A, x: torch.Tensor, topk_ids: torch.Tensor,
                 runtime_max_tokens_per_rank: int, workspace: torch.Tensor,
                 stream=None) -> None:
    """Route every routed copy of x into ``workspace`` ([ep, cap, H] bf16)."""
    T = x.shape[0] if x.dim() == 2 else 0
    _need(x, "x", torch.bfloat16, h.device_index, shape=(T, h.hidden))
    _need(topk_ids, "topk_ids", torch.int32, h.device_index, shape=(T, h.top_k))
    _need(workspace, "workspace", torch.bfloat16, h.device_index, numel=h.workspace_numel)
    _check(_fast().dispatch(h.addr, _ptr(x), _ptr(topk_ids), T, runtime_max_tokens_per_rank,
                            _ptr(workspace), _stream(stream, h.device_index)), "moe_dispatch")


def moe_dispatch_noalloc(h: MoeA2A, x: torch.Tensor, topk_ids: torch.Tensor,
                         runtime_max_tokens_per_rank: int, workspace: torch.Tensor,
                         stream=None) -> None:
    """moe_dispatch with the routing scratch taken from the library's static
    per-GPU array (no allocation anywhere in the call)."""
    T = x.shape[0] if x.dim() == 2 else 0
    _need(x, "x", torch.bfloat16, h.device_index, shape=(T, h.hidden))
    _need(topk_ids, "topk_ids", torch.int32, h.device_index, shape=(T, h.top_k))
    _need(workspace, "workspace", torch.bfloat16, h.device_index, numel=h.workspace_numel)
    _check(library().moe_dispatch_noalloc(h.ref, _ptr(x), _ptr(topk_ids), T,
                                          runtime_max_tokens_per_rank, _ptr(workspace),
                                          _stream(stream, h.device_index)), "moe_dispatch_noalloc")


def moe_dispatch_fp8(h: MoeA2A, x: torch.Tensor, topk_ids: torch.Tensor,
                     runtime_max_tokens_per_rank: int, workspace: torch.Tensor,
                     scales: torch.Tensor, stream=None) -> None:
    """Route every copy with an FP8 (e4m3) payload: codes into ``workspace``
    ([ep, cap, H] uint8), one fp32 scale per row into ``scales`` ([ep, cap])."""
    T = x.shape[0] if x.dim() == 2 else 0
    _need(x, "x", torch.bfloat16, h.device_index, shape=(T, h.hidden))
    _need(topk_ids, "topk_ids", torch.int32, h.device_index, shape=(T, h.top_k))
    _need(workspace, "workspace", torch.uint8, h.device_index, numel=h.workspace_numel)
    _need(scales, "scales", torch.float32, h.device_index, numel=h.ep_size * h.cap)
    _check(_fast().dispatch_fp8(h.addr, _ptr(x), _ptr(topk_ids), T, runtime_max_tokens_per_rank,
                                _ptr(workspace), _ptr(scales), _stream(stream, h.device_index)),
           "moe_dispatch_fp8")


def moe_combine(h: MoeA2A, expert_out: torch.Tensor, topk_weights: Optional[torch.Tensor] = None,
                weighted: Optional[bool] = None, out: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """out[t] = bf16(sum_j c_j * expert_out[slot(t, j)]), reduced once in fp32."""
    T = h.handle.num_tokens
    weighted = (topk_weights is not None) if weighted is None else bool(weighted)
    _need(expert_out, "expert_out", torch.bfloat16, h.device_index, numel=h.workspace_numel)
    if weighted:
        _need(topk_weights, "topk_weights", torch.float32, h.device_index, shape=(T, h.top_k))
    if out is None:
        out = torch.empty((T, h.hidden), dtype=torch.bfloat16, device=expert_out.device)
    _need(out, "out", torch.bfloat16, h.device_index, shape=(T, h.hidden))
    _check(_fast().combine(h.addr, _ptr(expert_out), _ptr(topk_weights) if weighted else None,
                           int(weighted), _ptr(out), _stream(stream, h.device_index)),
           "moe_combine")
    return out


def moe_combine_residual_rmsnorm(h: MoeA2A, expert_out: torch.Tensor,
                                 topk_weights: Optional[torch.Tensor], weighted: bool,
                                 residual: torch.Tensor, gamma: torch.Tensor, eps: float,
                                 residual_out: Optional[torch.Tensor] = None,
                                 normed: Optional[torch.Tensor] = None,
                                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Combine, add the residual and RMSNorm in one pass.

    Returns (residual_out, normed); ``residual_out`` may be ``residual``."""
    T, H = h.handle.num_tokens, h.hidden
    _need(expert_out, "expert_out", torch.bfloat16, h.device_index, numel=h.workspace_numel)
    if weighted:
        _need(topk_weights, "topk_weights", torch.float32, h.device_index, shape=(T, h.top_k))
    _need(residual, "residual", torch.bfloat16, h.device_index, shape=(T, H))
    _need(gamma, "gamma", torch.bfloat16, h.device_index, shape=(H,))
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if normed is None:
        normed = torch.empty_like(residual)
    _need(residual_out, "residual_out", torch.bfloat16, h.device_index, shape=(T, H))
    _need(normed, "normed", torch.bfloat16, h.device_index, shape=(T, H))
    _check(_fast().combine_residual_rmsnorm(
        h.addr, _ptr(expert_out), _ptr(topk_weights) if weighted else None,
        int(bool(weighted)), _ptr(residual), _ptr(residual_out), _ptr(gamma), float(eps),
        _ptr(normed), _stream(stream, h.device_index)), "moe_combine_residual_rmsnorm")
    return residual_out, normed


def moe_route_counts(h: MoeA2A, topk_ids: torch.Tensor, stream=None) -> torch.Tensor:
    """Per-region copy counts of a routing (for sizing max_tokens_per_rank)."""
    T = topk_ids.shape[0]
    _need(topk_ids, "topk_ids", torch.int32, h.device_index, shape=(T, h.top_k))
    _check(_fast().route_counts(h.addr, _ptr(topk_ids), T, _stream(stream, h.device_index)),
           "moe_route_counts")
    return h.counts


def moe_sync_status(h: MoeA2A, stream=None) -> Tuple[int, int]:
    """Wait for the stream; returns (code, status bits) and clears the bits."""
    bits = ctypes.c_int32(0)
    code = library().moe_sync_status(h.ref, _stream(stream, h.device_index), ctypes.byref(bits))
    if code == MOE_ERR_HIP or code == MOE_ERR_ARG:
        raise MoeError(code, "moe_sync_status")
    return code, bits.value


def moe_reset(h: MoeA2A) -> None:
    _check(library().moe_reset(h.ref), "moe_reset")


def _need_partials(partials: torch.Tensor) -> Tuple[int, int, int, int]:
    """(P, T, H, device index) of a [P, T, H] bf16 GPU tensor; the other
    tensors of the call must be on the same GPU."""
    if not isinstance(partials, torch.Tensor) or partials.dim() != 3:
        raise ValueError("partials must be a [P, T, H] tensor")
    if not partials.is_cuda:            # get_device() is -1 off the GPU
        raise ValueError("partials must be on the GPU")
    dev = partials.get_device()
    _need(partials, "partials", torch.bfloat16, dev)
    P, T, H = partials.shape
    return P, T, H, dev


def moe_partials_reduce(partials: torch.Tensor, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Sum of P partial hidden states [P, T, H] (the reduction stage of an
    all-reduce, on one GPU): out = bf16(fp32 sum in rank order)."""
    P, T, H, dev = _need_partials(partials)
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=partials.device)
    _need(out, "out", torch.bfloat16, dev, shape=(T, H))
    _check(_fast().partials_reduce(_ptr(partials), P, T, H, _ptr(out), _stream(stream, dev)),
           "moe_partials_reduce")
    return out


def moe_partials_reduce_residual_rmsnorm(partials: torch.Tensor, residual: torch.Tensor,
                                         gamma: torch.Tensor, eps: float,
                                         residual_out: Optional[torch.Tensor] = None,
                                         normed: Optional[torch.Tensor] = None,
                                         stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Sum of the partials, residual add and RMSNorm in one pass.

    Returns (residual_out, normed); ``residual_out`` may be ``residual``."""
    P, T, H, dev = _need_partials(partials)
    _need(residual, "residual", torch.bfloat16, dev, shape=(T, H))
    _need(gamma, "gamma", torch.bfloat16, dev, shape=(H,))
    if residual_out is None:
        residual_out = torch.empty_like(residual)
    if normed is None:
        normed = torch.empty_like(residual)
    _need(residual_out, "residual_out", torch.bfloat16, dev, shape=(T, H))
    _need(normed, "normed", torch.bfloat16, dev, shape=(T, H))
    _check(_fast().partials_reduce_residual_rmsnorm(
        _ptr(partials), P, T, H, _ptr(residual), _ptr(residual_out), _ptr(gamma), float(eps),
        _ptr(normed), _stream(stream, dev)), "moe_partials_reduce_residual_rmsnorm")
    return residual_out, normed


__all__ = [
    "MoeA2A", "MoeError", "MoeHandle", "library", "moe_dispatch", "moe_dispatch_noalloc",
    "moe_dispatch_fp8", "moe_combine",
    "moe_combine_residual_rmsnorm", "moe_route_counts", "moe_sync_status", "moe_reset",
    "moe_output_is_reduced", "moe_strerror", "moe_workspace_bytes", "moe_scratch_bytes",
    "moe_partials_reduce", "moe_partials_reduce_residual_rmsnorm", "moe_last_hip_error",
]
