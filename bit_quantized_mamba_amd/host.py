"""ctypes binding of libdfssm_host.so (include/dfssm_host.h): the host CPU
backend of the DF-SSM decode step.  Argument marshalling only; numpy arrays
in host memory.  A separate engine, selected explicitly: the device library
never falls back to it."""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import numpy as np

from . import GLOBAL_KINDS, LAYER_KINDS, _Shapes
from ._lib import DfssmConfig, DfssmError

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB_PATH = os.path.join(_HERE, "libdfssm_host.so")

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t

EXPORTS = {
    "dfssm_host_last_error": [],
    "dfssm_host_create": [ctypes.POINTER(DfssmConfig), _i32, ctypes.POINTER(_p)],
    "dfssm_host_destroy": [_p],
    "dfssm_host_set_isa": [_p, _i32],
    "dfssm_host_get_isa": [_p, ctypes.POINTER(_i32)],
    "dfssm_host_load_synthetic": [_p, ctypes.c_uint64],
    "dfssm_host_set_tensor": [_p, _i32, _i32, _p, _sz],
    "dfssm_host_get_tensor": [_p, _i32, _i32, _p, _sz],
    "dfssm_host_reset_state": [_p, _i32],
    "dfssm_host_get_state": [_p, _i32, _p, _p],
    "dfssm_host_set_state": [_p, _i32, _p, _p],
    "dfssm_host_decode_step": [_p, _p, _i32, _p, _p],
    "dfssm_host_trace_step": [_p, _p, _i32, _p, _p, _p, _p, _p, _p, _p],
    "dfssm_host_generate": [_p, _p, _i32, _i32, _p],
    "dfssm_host_prefill": [_p, _p, _i32, _i32, _p, _p],
    "dfssm_host_copy_rate": [_p, _sz, _i32, ctypes.POINTER(ctypes.c_double)],
}
_RESTYPE = {"dfssm_host_last_error": ctypes.c_char_p, "dfssm_host_destroy": None}

_lib = None


def load() -> ctypes.CDLL:
    """Load the host library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(HOST_LIB_PATH):
            raise ImportError(f"{HOST_LIB_PATH} is missing: build it with `python -m bit_quantized_mamba_amd.build`")
        L = ctypes.CDLL(HOST_LIB_PATH)
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
        raise DfssmError(name, rc, L.dfssm_host_last_error().decode())


def _ptr(a: Optional[np.ndarray]) -> Optional[int]:
    return None if a is None else a.ctypes.data


def _i32_array(a, ndim: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.int32)
    if a.ndim != ndim:
        raise ValueError(f"token array must have {ndim} dimension(s)")
    return a


class HostEngine(_Shapes):
    """A DF-SSM model held in host memory: weights, the recurrent state of
    `max_batch` sequence slots and the workspace, owned by the host library."""

    ISAS = {"auto": 0, "portable": 1, "avx512vnni": 2}

    def __init__(self, n_layer: int, d_model: int, d_inner: int, d_state: int, headdim: int, vocab: int,
                 d_conv: int = 4, rank: int = 16, max_batch: int = 1, threads: int = 0, norm_eps: float = 1e-5):
        self.cfg = DfssmConfig(n_layer, d_model, d_inner, d_state, headdim, vocab, d_conv, rank, max_batch, norm_eps, 0)
        self.n_layer, self.d_model, self.d_inner, self.d_state = n_layer, d_model, d_inner, d_state
        self.headdim, self.vocab, self.d_conv, self.rank, self.max_batch = headdim, vocab, d_conv, rank, max_batch
        self.n_heads = d_inner // headdim
        self.conv_dim = d_inner + 2 * d_state
        self.d_in_proj = 2 * d_inner + 2 * d_state + self.n_heads
        h = _p()
        call("dfssm_host_create", ctypes.byref(self.cfg), threads, ctypes.byref(h))
        self._h = h

    @classmethod
    def from_shape(cls, s, max_batch: int = 1, threads: int = 0) -> "HostEngine":
        return cls(s.n_layer, s.d_model, s.d_inner, s.d_state, s.headdim, s.vocab, s.d_conv, s.rank,
                   max_batch=max_batch, threads=threads)

    def close(self) -> None:
        if getattr(self, "_h", None):
            load().dfssm_host_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- instruction path ------------------------------------------------------
    def set_isa(self, name: str) -> None:
        call("dfssm_host_set_isa", self._h, self.ISAS[name])

    @property
    def isa(self) -> str:
        v = _i32()
        call("dfssm_host_get_isa", self._h, ctypes.byref(v))
        return {k: n for n, k in self.ISAS.items()}[v.value]

    # -- weights ---------------------------------------------------------------
    def load_synthetic(self, seed: int) -> None:
        call("dfssm_host_load_synthetic", self._h, seed)

    def set_tensor(self, layer: int, kind: str, value: np.ndarray) -> None:
        shp, dt = self._tensor_shape(layer, kind)
        a = np.ascontiguousarray(value, dtype=dt)
        if a.shape != shp:
            raise ValueError(f"{kind}: shape {a.shape}, expected {shp}")
        call("dfssm_host_set_tensor", self._h, layer, self._kind_id(layer, kind), a.ctypes.data, a.nbytes)

    def get_tensor(self, layer: int, kind: str) -> np.ndarray:
        shp, dt = self._tensor_shape(layer, kind)
        a = np.empty(shp, dtype=dt)
        call("dfssm_host_get_tensor", self._h, layer, self._kind_id(layer, kind), a.ctypes.data, a.nbytes)
        return a

    def set_weights(self, weights) -> None:
        for l, lay in enumerate(weights["layers"]):
            for k in LAYER_KINDS:
                self.set_tensor(l, k, lay[k])
        for k in GLOBAL_KINDS:
            if k in weights:
                self.set_tensor(-1, k, weights[k])

    # -- state -----------------------------------------------------------------
    def reset_state(self, batch: Optional[int] = None) -> None:
        call("dfssm_host_reset_state", self._h, self.max_batch if batch is None else batch)

    def get_state(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        conv = np.empty((self.n_layer, self.conv_dim, self.d_conv - 1), dtype=np.float32)
        ssm = np.empty((self.n_layer, self.n_heads, self.headdim, self.d_state), dtype=np.float32)
        call("dfssm_host_get_state", self._h, seq, conv.ctypes.data, ssm.ctypes.data)
        return conv, ssm

    def set_state(self, seq: int, conv: Optional[np.ndarray] = None, ssm: Optional[np.ndarray] = None) -> None:
        c = None if conv is None else np.ascontiguousarray(conv, dtype=np.float32)
        s = None if ssm is None else np.ascontiguousarray(ssm, dtype=np.float32)
        if c is not None and c.shape != (self.n_layer, self.conv_dim, self.d_conv - 1):
            raise ValueError("conv state shape")
        if s is not None and s.shape != (self.n_layer, self.n_heads, self.headdim, self.d_state):
            raise ValueError("ssm state shape")
        call("dfssm_host_set_state", self._h, seq, _ptr(c), _ptr(s))

    # -- compute ---------------------------------------------------------------
    def decode_step(self, tok) -> Tuple[np.ndarray, np.ndarray]:
        t = _i32_array(tok, 1)
        B = t.shape[0]
        logits = np.empty((B, self.vocab), dtype=np.float32)
        nxt = np.empty((B,), dtype=np.int32)
        call("dfssm_host_decode_step", self._h, t.ctypes.data, B, logits.ctypes.data, nxt.ctypes.data)
        return logits, nxt

    def trace_step(self, tok, want_acc: bool = True) -> Dict[str, np.ndarray]:
        """Decode step recording h [L+1][B][d_model], q1 [L][B][d_model], q2 [L][B][d_inner], qf [B][d_model],
        logits [B][vocab] and (with want_acc) acc1 [L][B][d_in_proj], acc2 [L][B][d_model]."""
        t = _i32_array(tok, 1)
        B, L = t.shape[0], self.n_layer
        tr = {"h": np.empty((L + 1, B, self.d_model), np.float32), "q1": np.empty((L, B, self.d_model), np.int8),
              "q2": np.empty((L, B, self.d_inner), np.int8), "qf": np.empty((B, self.d_model), np.int8),
              "logits": np.empty((B, self.vocab), np.float32)}
        if want_acc:
            tr["acc1"] = np.empty((L, B, self.d_in_proj), np.int32)
            tr["acc2"] = np.empty((L, B, self.d_model), np.int32)
        call("dfssm_host_trace_step", self._h, t.ctypes.data, B, tr["h"].ctypes.data, tr["q1"].ctypes.data,
             tr["q2"].ctypes.data, tr["qf"].ctypes.data, tr["logits"].ctypes.data, _ptr(tr.get("acc1")),
             _ptr(tr.get("acc2")))
        return tr

    def generate(self, tok: np.ndarray, n_steps: int) -> np.ndarray:
        """Greedy decode n_steps from tok (int32 [B], updated in place to the last token)."""
        if not (isinstance(tok, np.ndarray) and tok.dtype == np.int32 and tok.ndim == 1 and tok.flags.c_contiguous):
            raise ValueError("tok must be a contiguous int32 numpy array [B] (it receives the last tokens)")
        B = tok.shape[0]
        out = np.empty((n_steps, B), dtype=np.int32)
        call("dfssm_host_generate", self._h, tok.ctypes.data, B, n_steps, out.ctypes.data)
        return out

    def prefill(self, tok) -> Tuple[np.ndarray, np.ndarray]:
        t = _i32_array(tok, 2)
        B, T = t.shape
        logits = np.empty((B, self.vocab), dtype=np.float32)
        nxt = np.empty((B,), dtype=np.int32)
        call("dfssm_host_prefill", self._h, t.ctypes.data, B, T, logits.ctypes.data, nxt.ctypes.data)
        return logits, nxt

    def copy_rate(self, nbytes: int = 1 << 30, iters: int = 5) -> float:
        """Measured host copy rate with this engine's threads, GB/s (read + write)."""
        v = ctypes.c_double()
        call("dfssm_host_copy_rate", self._h, nbytes, iters, ctypes.byref(v))
        return v.value
