"""ctypes binding of libdfssm.so (include/dfssm.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdfssm.so")

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class DfssmConfig(ctypes.Structure):
    _fields_ = [("n_layer", ctypes.c_int32), ("d_model", ctypes.c_int32), ("d_inner", ctypes.c_int32),
                ("d_state", ctypes.c_int32), ("headdim", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("d_conv", ctypes.c_int32), ("lora_rank", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("max_chunk_rows", ctypes.c_int32)]


# (name, argtypes); every function returns int32 status unless listed in _RESTYPE
EXPORTS = {
    "dfssm_version": [],
    "dfssm_last_error": [_p],
    "dfssm_arena_bytes": [ctypes.POINTER(DfssmConfig), ctypes.POINTER(_sz)],
    "dfssm_create": [ctypes.POINTER(DfssmConfig), _i32, _p, _sz, ctypes.POINTER(_p)],
    "dfssm_destroy": [_p],
    "dfssm_device_bytes": [_p, ctypes.POINTER(_sz)],
    "dfssm_set_path": [_p, _i32],
    "dfssm_load_synthetic": [_p, ctypes.c_uint64, _p],
    "dfssm_set_tensor": [_p, _i32, _i32, _p, _sz],
    "dfssm_get_tensor": [_p, _i32, _i32, _p, _sz],
    "dfssm_reset_state": [_p, _i32, _p],
    "dfssm_get_state": [_p, _i32, _p, _p],
    "dfssm_set_state": [_p, _i32, _p, _p],
    "dfssm_decode_step": [_p, _p, _i32, _p, _p, _p],
    "dfssm_generate": [_p, _p, _i32, _i32, _p, _i32, _p],
    "dfssm_prefill": [_p, _p, _i32, _i32, _p, _p, _p],
    "dfssm_layer_step": [_p, _i32, _p, _p, _i32, _p, _p, _p],
    "dfssm_layer_step_f16": [_p, _i32, _p, _p, _i32, _p, _p, _p],
    "dfssm_trace_step": [_p, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _p],
    "dfssm_trace_prefill": [_p, _p, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p],
    "dfssm_check_device": [_p, _p],
    "dfssm_state_pack": [_p, _i32, _i32, _p, _p, _p],
    "dfssm_state_unpack": [_p, _i32, _i32, _p, _p, _p],
    "dfssm_state_roundtrip": [_p, _i32, _i32, _p],
    "dfssm_k_density_encode": [_p, _i32, _i32, _p, _p, _p],
    "dfssm_k_density_decode": [_p, _p, _i32, _i32, _p, _p],
    "dfssm_profile_persistent": [_p, _p, _i32, _p, _i32, _p],
    "dfssm_time_kernel": [_p, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_float), _p],
    "dfssm_k_quant": [_p, _i32, _i32, _p, _p, _p],
    "dfssm_k_proj": [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _p, _p, _i32, _p, _p, _p],
    "dfssm_k_gemm": [_p, _p, _p, _p, _p, _p, _i32, _i32, _p, _p, _i32, _p, _p, _p],
    "dfssm_k_gemm_noalloc": [_p, _p, _p, _p, _p, _p, _i32, _i32, _p, _p, _i32, _p, _p, _p],
}
_RESTYPE = {"dfssm_version": ctypes.c_char_p, "dfssm_last_error": ctypes.c_char_p, "dfssm_destroy": None}

_lib = None


class DfssmError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_mamba_amd.build` "
                              "(hipcc, gfx950); there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in EXPORTS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _RESTYPE.get(name, ctypes.c_int32)
        _lib = L
    return _lib


def call(name: str, *args) -> None:
    L = load()
    rc = getattr(L, name)(*args)
    if rc != 0:
        raise DfssmError(name, rc, L.dfssm_last_error(None).decode())
