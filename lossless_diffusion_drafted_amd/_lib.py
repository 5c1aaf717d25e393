"""ctypes binding of libuno.so: argument marshalling only.

Every computation runs in the HIP kernels behind the C ABI declared in
include/uno.h. PyTorch supplies device memory and the current HIP stream. If the
library has not been built, every call raises: there is no fallback path.
"""

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libuno.so")

UNO_OK = 0
UNO_ERR_INVALID_ARG = 1
UNO_ERR_UNSUPPORTED = 2
UNO_ERR_WORKSPACE = 3
UNO_ERR_HIP = 4
UNO_DTYPE_F32 = 0
UNO_DTYPE_BF16 = 1

FLAG_TIE_ACCEPT = 1
FLAG_TIE_TOPP_P = 2
FLAG_TIE_TOPP_Q = 4
FLAG_TIE_ICDF = 8
FLAG_Q_ZERO = 16
FLAG_RES_ZERO = 32
FLAG_OVERFLOW = 64
FLAG_TIE_MASK = FLAG_TIE_ACCEPT | FLAG_TIE_TOPP_P | FLAG_TIE_TOPP_Q | FLAG_TIE_ICDF

EXPORTS = [
    "uno_status_string", "uno_last_error", "uno_abi_version", "uno_workspace_init",
    "uno_verify_block_workspace", "uno_verify_block", "uno_verify_block_noalloc", "uno_draft_sample",
    "uno_tv_loss_workspace", "uno_tv_loss_fwd_bwd",
    "uno_gated_lora_linear_workspace", "uno_gated_lora_linear",
    "uno_gated_lora_linear_bwd_workspace", "uno_gated_lora_linear_bwd",
    "uno_forward_workspace", "uno_forward", "uno_decode_step_workspace", "uno_decode_step",
    "uno_ar_step_workspace", "uno_ar_step",
]


class SamplingParams(ctypes.Structure):
    """uno_sampling_params (include/uno.h)."""
    _fields_ = [("temperature", ctypes.c_double), ("top_p", ctypes.c_double),
                ("top_k", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class UnoModel(ctypes.Structure):
    """uno_model (include/uno.h)."""
    _fields_ = [("hidden", ctypes.c_int), ("kv_width", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("ffn", ctypes.c_int), ("vocab", ctypes.c_int), ("layers", ctypes.c_int),
                ("rank", ctypes.c_int), ("lora_scale", ctypes.c_float),
                ("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("weights", ctypes.POINTER(ctypes.c_void_p)), ("lora_a", ctypes.POINTER(ctypes.c_void_p)),
                ("lora_b", ctypes.POINTER(ctypes.c_void_p))]


class UnoError(RuntimeError):
    def __init__(self, status, fn, detail):
        super().__init__(f"{fn} returned {status}: {detail}")
        self.status = status


_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


def load():
    """Load libuno.so once and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m lossless_diffusion_drafted_amd.build` "
                "(the HIP library is the only implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        sig = {
            "uno_status_string": (ctypes.c_char_p, [_I]),
            "uno_last_error": (ctypes.c_char_p, []),
            "uno_abi_version": (_I, []),
            "uno_workspace_init": (_I, [_P, _SZ, _P]),
            "uno_verify_block_workspace": (_SZ, [_I, _I, _I]),
            "uno_verify_block": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, SamplingParams,
                                      _P, _P, _P, _P, _P, _P, _SZ, _P]),
            "uno_verify_block_noalloc": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, SamplingParams,
                                              _P, _P, _P, _P, _P, _P]),
            "uno_draft_sample": (_I, [_P, _I, _P, _P, _I, _I, _I, SamplingParams, _P, _P, _P]),
            "uno_tv_loss_workspace": (_SZ, [_I, _I]),
            "uno_tv_loss_fwd_bwd": (_I, [_P, _P, _I, _P, _I, _I, ctypes.c_float, _P, _P, _P,
                                         _P, _SZ, _P]),
            "uno_gated_lora_linear_workspace": (_SZ, [_I, _I, _I, _I]),
            "uno_gated_lora_linear": (_I, [_P, _P, _P, _P, _P, ctypes.c_float, _P, _I, _I, _I,
                                           _I, _P, _SZ, _P]),
            "uno_gated_lora_linear_bwd_workspace": (_SZ, [_I, _I, _I, _I]),
            "uno_gated_lora_linear_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _I,
                                               _I, _I, _I, _P, _SZ, _P]),
            "uno_forward_workspace": (_SZ, [_P, _I]),
            "uno_forward": (_I, [_P, _P, _P, _I, _I, _P, _P, _SZ, _P]),
            "uno_decode_step_workspace": (_SZ, [_P, _I, _I]),
            "uno_decode_step": (_I, [_P, _I, _I, _I, _I, SamplingParams, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _P, _SZ, _P]),
            "uno_ar_step_workspace": (_SZ, [_P, _I]),
            "uno_ar_step": (_I, [_P, _I, _I, SamplingParams, _P, _P, _P, _P, _P, _P, _SZ, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
        return lib


def check(status, fn):
    if status != UNO_OK:
        lib = load()
        raise UnoError(lib.uno_status_string(status).decode(), fn, lib.uno_last_error().decode())


# --- torch marshalling helpers --------------------------------------------------

def _torch():
    import torch
    return torch


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_handle(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return UNO_DTYPE_BF16
    if t.dtype == torch.float32:
        return UNO_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def require(t, name, dtype=None, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


class Workspaces:
    """Zero-initialised device workspaces, one per (device, stream, purpose).

    Each library call leaves its workspace valid for the next call, so a buffer is
    cleared only when it is first allocated or grown."""

    def __init__(self):
        self._bufs = {}
        self._lock = threading.Lock()

    def get(self, device, stream, purpose, nbytes):
        torch = _torch()
        nbytes = max(256, (int(nbytes) + 255) // 256 * 256)
        key = (str(device), stream.value, purpose)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() < nbytes:
                buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
                check(load().uno_workspace_init(ptr(buf), nbytes, stream), "uno_workspace_init")
                self._bufs[key] = buf
            return buf


WORKSPACES = Workspaces()
