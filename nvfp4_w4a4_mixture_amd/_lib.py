"""ctypes loader for libmoe_nvfp4.so (the C ABI declared in include/moe_nvfp4.h).

PyTorch is imported first so that the library binds to the HIP runtime torch
already loaded (same soname), and torch's device pointers and streams are
valid in the library's calls.  There is no fallback: if the library is not
built, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first)

# MOE_NVFP4_LIB selects another build of the same library (the host-sanitized one, for example)
LIB_PATH = os.environ.get("MOE_NVFP4_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                           "libmoe_nvfp4.so")

MOE_OK = 0
ABI_VERSION = 3  # MOE_NVFP4_ABI_VERSION these signatures follow
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN", 4: "MOE_ERR_WORKSPACE",
                5: "MOE_ERR_DEVICE", 6: "MOE_ERR_LAUNCH"}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/moe_nvfp4.h
SIGNATURES = {
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (_i32, []),
    "moe_route_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "moe_route": (_i32, [_p, _i64, _i64, _i64, _p, _p, _i64, _i64, _f32, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_route_quantize": (_i32, [_p, _i64, _i64, _i64, _p, _p, _i64, _i64, _f32, _p, _p, _p, _p, _p, _p, _p, _p,
                                  _p, _sz, _p]),
    "nvfp4_quantize_act": (_i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "nvfp4_quantize_weights": (_i32, [_p, _i64, _i64, _i64, _p, _p, _p, _p]),
    "moe_ffn_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "moe_ffn_stage_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "moe_nvfp4_grouped_ffn": (_i32, [_p, _p, _p, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                     _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_nvfp4_grouped_ffn_noalloc": (_i32, [_p, _p, _p, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                             _p, _p, _p, _p, _p, _p, _p]),
    "moe_nvfp4_gate_up_swiglu": (_i32, [_p, _p, _p, _i64, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _p, _p,
                                        _p, _p, _p, _sz, _p]),
    "moe_nvfp4_down_scatter": (_i32, [_p, _p, _p, _i64, _i64, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p,
                                      _p, _p, _p, _sz, _p]),
    "moe_combine": (_i32, [_p, _p, _i64, _i64, _i64, _i32, _p, _p]),
    "reap_saliency": (_i32, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p]),
    "moe_combine_reap": (_i32, [_p, _p, _i64, _i64, _i64, _i32, _p, _p, _p, _p, _p, _i64, _p, _p]),
    "reap_prune_select": (_i32, [_p, _i64, _i64, _p, _p]),
    "moe_gather_experts": (_i32, [_p, _i64, _i64, _p, _i64, _p, _p]),
    "moe_shared_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "moe_shared_expert": (_i32, [_p, _i64, _i64, _i64, _p, _p, _i64, _p, _p, _sz, _p]),
    "moe_shared_gate_up": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _p, _p, _sz, _p]),
    "moe_shared_down": (_i32, [_p, _i64, _i64, _p, _i64, _p, _p, _sz, _p]),
    "moe_combine_block": (_i32, [_p, _p, _p, _i64, _i64, _i64, _i32, _p, _p]),
    "hadamard_rotate_bf16": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _p, _i64, _p]),
    "moe_nvfp4_prepack_weights": (_i32, [_p, _p, _i64, _i64, _i64, _i32, _p, _p, _p]),
    "moe_nvfp4_unpack_weights": (_i32, [_p, _p, _i64, _i64, _i64, _i32, _p, _p, _p]),
}


class MoEError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m nvfp4_w4a4_mixture_amd.build` "
                           "(there is no CPU fallback for the HIP path)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    version = lib.moe_abi_version()
    if version != ABI_VERSION:
        raise RuntimeError(f"{path} implements ABI version {version}, this binding expects {ABI_VERSION}; rebuild it")
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def check(status: int, fn: str) -> None:
    if status != MOE_OK:
        raise MoEError(status, fn, lib().moe_last_error().decode())
