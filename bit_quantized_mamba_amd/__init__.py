"""DF-SSM 1-bit-scaffold Mamba-2 decode on AMD Instinct MI355X (gfx950).

A thin Python face of the C-ABI library libdfssm.so (include/dfssm.h).  PyTorch
supplies device memory and streams; every step of the model runs in the
library's HIP kernels.  If the library is missing, importing the binding
raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import numpy as np

from . import _lib
from ._lib import DfssmConfig, DfssmError, call

LAYER_KINDS = ["in_bits", "in_sw", "in_A", "in_sA", "in_B", "in_sB", "out_bits", "out_sw", "out_A", "out_sA",
               "out_B", "out_sB", "conv_w", "conv_b", "A_log", "dt_bias", "D", "norm_w", "gnorm_w"]
GLOBAL_KINDS = ["E", "sE", "final_norm"]

__all__ = ["Engine", "DfssmError", "k_quant", "k_proj", "k_gemm", "k_gemm_noalloc", "k_density_encode",
           "k_density_decode", "version", "LAYER_KINDS", "GLOBAL_KINDS"]


def version() -> str:
    return _lib.load().dfssm_version().decode()


def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dp(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class _Shapes:
    """Shapes and kind ids of the weight tensors (canonical layouts of include/dfssm.h), from the
    dimensions an engine holds as attributes."""

    def _tensor_shape(self, layer: int, kind: str):
        r = self.rank
        if layer < 0:
            return {"E": ((self.vocab, self.d_model), np.int8), "sE": ((self.vocab,), np.float32),
                    "final_norm": ((self.d_model,), np.float32)}[kind]
        dp, dm, di, cd, H = self.d_in_proj, self.d_model, self.d_inner, self.conv_dim, self.n_heads
        return {"in_bits": ((dp, dm // 32), np.uint32), "in_sw": ((dp,), np.float32), "in_A": ((r, dm), np.int8),
                "in_sA": ((r,), np.float32), "in_B": ((dp, r), np.int8), "in_sB": ((dp,), np.float32),
                "out_bits": ((dm, di // 32), np.uint32), "out_sw": ((dm,), np.float32),
                "out_A": ((r, di), np.int8), "out_sA": ((r,), np.float32), "out_B": ((dm, r), np.int8),
                "out_sB": ((dm,), np.float32), "conv_w": ((cd, self.d_conv), np.float32),
                "conv_b": ((cd,), np.float32), "A_log": ((H,), np.float32), "dt_bias": ((H,), np.float32),
                "D": ((H,), np.float32), "norm_w": ((dm,), np.float32), "gnorm_w": ((di,), np.float32)}[kind]

    def _kind_id(self, layer: int, kind: str) -> int:
        return GLOBAL_KINDS.index(kind) if layer < 0 else LAYER_KINDS.index(kind)


class Engine(_Shapes):
    """A DF-SSM model held on one GPU: weights, the recurrent state of
    `max_batch` sequence slots and the workspace, owned by the library."""

    def __init__(self, n_layer: int, d_model: int, d_inner: int, d_state: int, headdim: int, vocab: int,
                 d_conv: int = 4, rank: int = 16, max_batch: int = 1, device: int = 0, norm_eps: float = 1e-5,
                 max_chunk_rows: int = 0, arena=None):
        """arena: optional uint8 CUDA tensor of at least arena_bytes(...) bytes (256-byte aligned) that
        holds everything the context needs; the engine keeps a reference to it until close()."""
        self.cfg = DfssmConfig(n_layer, d_model, d_inner, d_state, headdim, vocab, d_conv, rank, max_batch, norm_eps,
                               max_chunk_rows)
        self.n_layer, self.d_model, self.d_inner, self.d_state = n_layer, d_model, d_inner, d_state
        self.headdim, self.vocab, self.d_conv, self.rank, self.max_batch = headdim, vocab, d_conv, rank, max_batch
        self.n_heads = d_inner // headdim
        self.conv_dim = d_inner + 2 * d_state
        self.d_in_proj = 2 * d_inner + 2 * d_state + self.n_heads
        self.device = device
        self._arena = arena
        h = ctypes.c_void_p()
        if arena is None:
            call("dfssm_create", ctypes.byref(self.cfg), device, None, 0, ctypes.byref(h))
        else:
            call("dfssm_create", ctypes.byref(self.cfg), device, arena.data_ptr(),
                 arena.numel() * arena.element_size(), ctypes.byref(h))
        self._h = h

    @staticmethod
    def arena_bytes(n_layer: int, d_model: int, d_inner: int, d_state: int, headdim: int, vocab: int,
                    d_conv: int = 4, rank: int = 16, max_batch: int = 1, norm_eps: float = 1e-5,
                    max_chunk_rows: int = 0) -> int:
        """Device bytes an engine of this configuration needs in a caller-provided arena."""
        cfg = DfssmConfig(n_layer, d_model, d_inner, d_state, headdim, vocab, d_conv, rank, max_batch, norm_eps,
                          max_chunk_rows)
        n = ctypes.c_size_t()
        call("dfssm_arena_bytes", ctypes.byref(cfg), ctypes.byref(n))
        return n.value

    @classmethod
    def from_shape(cls, s, max_batch: int = 1, device: int = 0, max_chunk_rows: int = 0, arena=None) -> "Engine":
        return cls(s.n_layer, s.d_model, s.d_inner, s.d_state, s.headdim, s.vocab, s.d_conv, s.rank,
                   max_batch=max_batch, device=device, max_chunk_rows=max_chunk_rows, arena=arena)

    def close(self) -> None:
        if getattr(self, "_h", None):
            _lib.load().dfssm_destroy(self._h)
            self._h = None
        self._arena = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- weights -----------------------------------------------------------
    def load_synthetic(self, seed: int, stream=None) -> None:
        call("dfssm_load_synthetic", self._h, ctypes.c_uint64(seed), _stream(stream))

    def set_tensor(self, layer: int, kind: str, value: np.ndarray) -> None:
        shp, dt = self._tensor_shape(layer, kind)
        a = np.ascontiguousarray(value, dtype=dt)
        if a.shape != shp:
            raise ValueError(f"{kind}: shape {a.shape}, expected {shp}")
        call("dfssm_set_tensor", self._h, layer, self._kind_id(layer, kind), a.ctypes.data, a.nbytes)

    def get_tensor(self, layer: int, kind: str) -> np.ndarray:
        shp, dt = self._tensor_shape(layer, kind)
        a = np.empty(shp, dtype=dt)
        call("dfssm_get_tensor", self._h, layer, self._kind_id(layer, kind), a.ctypes.data, a.nbytes)
        return a

    def set_weights(self, weights) -> None:
        """Upload a whole model given as {"layers": [dict per layer], "E", "sE", "final_norm"}."""
        for l, lay in enumerate(weights["layers"]):
            for k in LAYER_KINDS:
                self.set_tensor(l, k, lay[k])
        for k in GLOBAL_KINDS:
            if k in weights:
                self.set_tensor(-1, k, weights[k])

    # -- state -------------------------------------------------------------
    def reset_state(self, batch: Optional[int] = None, stream=None) -> None:
        call("dfssm_reset_state", self._h, batch or self.max_batch, _stream(stream))

    def get_state(self, seq: int) -> Tuple[np.ndarray, np.ndarray]:
        conv = np.empty((self.n_layer, self.conv_dim, self.d_conv - 1), dtype=np.float32)
        ssm = np.empty((self.n_layer, self.n_heads, self.headdim, self.d_state), dtype=np.float32)
        call("dfssm_get_state", self._h, seq, conv.ctypes.data, ssm.ctypes.data)
        return conv, ssm

    def set_state(self, seq: int, conv: Optional[np.ndarray], ssm: Optional[np.ndarray]) -> None:
        c = None if conv is None else np.ascontiguousarray(conv, dtype=np.float32)
        s = None if ssm is None else np.ascontiguousarray(ssm, dtype=np.float32)
        if c is not None and c.shape != (self.n_layer, self.conv_dim, self.d_conv - 1):
            raise ValueError("conv state shape")
        if s is not None and s.shape != (self.n_layer, self.n_heads, self.headdim, self.d_state):
            raise ValueError("ssm state shape")
        call("dfssm_set_state", self._h, seq, None if c is None else c.ctypes.data,
             None if s is None else s.ctypes.data)

    # -- compute -----------------------------------------------------------
    def _check_tok(self, tok, ndim: int):
        torch = _torch()
        if tok.dtype != torch.int32 or not tok.is_cuda or not tok.is_contiguous() or tok.dim() != ndim:
            raise ValueError(f"tokens must be a contiguous {ndim}-D int32 CUDA tensor")

    def decode_step(self, tok, logits=None, next_tok=None, stream=None):
        torch = _torch()
        self._check_tok(tok, 1)
        B = tok.shape[0]
        if logits is None:
            logits = torch.empty((B, self.vocab), dtype=torch.float32, device=tok.device)
        if next_tok is None:
            next_tok = torch.empty((B,), dtype=torch.int32, device=tok.device)
        call("dfssm_decode_step", self._h, _dp(tok), B, _dp(logits), _dp(next_tok), _stream(stream))
        return logits, next_tok

    def generate(self, tok, n_steps: int, out=None, use_graph: bool = True, stream=None):
        """Greedy decode n_steps from tok ([B] int32, updated in place to the last token)."""
        torch = _torch()
        self._check_tok(tok, 1)
        B = tok.shape[0]
        if out is None:
            out = torch.empty((n_steps, B), dtype=torch.int32, device=tok.device)
        call("dfssm_generate", self._h, _dp(tok), B, n_steps, _dp(out), int(use_graph), _stream(stream))
        return out

    def prefill(self, tok, want_logits: bool = True, stream=None):
        torch = _torch()
        self._check_tok(tok, 2)
        B, T = tok.shape
        logits = torch.empty((B, self.vocab), dtype=torch.float32, device=tok.device) if want_logits else None
        nxt = torch.empty((B,), dtype=torch.int32, device=tok.device)
        call("dfssm_prefill", self._h, _dp(tok), B, T, _dp(logits), _dp(nxt), _stream(stream))
        return logits, nxt

    def layer_step(self, layer: int, h_in, h_out=None, want_codes: bool = False, stream=None):
        """One layer on h_in ([B][d_model] fp32). Returns h_out, or (h_out, q1, q2) with want_codes."""
        torch = _torch()
        if h_in.dtype != torch.float32 or not h_in.is_cuda or not h_in.is_contiguous():
            raise ValueError("h_in must be a contiguous fp32 CUDA tensor [B][d_model]")
        B = h_in.shape[0]
        if h_out is None:
            h_out = torch.empty_like(h_in)
        q1 = torch.empty((B, self.d_model), dtype=torch.int8, device=h_in.device) if want_codes else None
        q2 = torch.empty((B, self.d_inner), dtype=torch.int8, device=h_in.device) if want_codes else None
        call("dfssm_layer_step", self._h, layer, _dp(h_in), _dp(h_out), B, _dp(q1), _dp(q2), _stream(stream))
        return (h_out, q1, q2) if want_codes else h_out

    def layer_step_f16(self, layer: int, h_in, h_out=None, want_codes: bool = False, stream=None):
        """layer_step with fp16 input activations h_in ([B][d_model] float16, upcast exactly on the device)."""
        torch = _torch()
        if h_in.dtype != torch.float16 or not h_in.is_cuda or not h_in.is_contiguous():
            raise ValueError("h_in must be a contiguous fp16 CUDA tensor [B][d_model]")
        B = h_in.shape[0]
        if h_out is None:
            h_out = torch.empty((B, self.d_model), dtype=torch.float32, device=h_in.device)
        q1 = torch.empty((B, self.d_model), dtype=torch.int8, device=h_in.device) if want_codes else None
        q2 = torch.empty((B, self.d_inner), dtype=torch.int8, device=h_in.device) if want_codes else None
        call("dfssm_layer_step_f16", self._h, layer, _dp(h_in), _dp(h_out), B, _dp(q1), _dp(q2), _stream(stream))
        return (h_out, q1, q2) if want_codes else h_out

    def trace_step(self, tok, want_acc: bool = True, stream=None):
        """Decode step recording the residual stream per layer, every int8 activation code and
        (with want_acc) the exact int32 scaffold sums of every projection row.

        Returns dict(h=[L+1][B][d_model], q1=[L][B][d_model], q2=[L][B][d_inner], qf=[B][d_model], logits,
        acc1=[L][B][d_in_proj], acc2=[L][B][d_model])."""
        torch = _torch()
        self._check_tok(tok, 1)
        B = tok.shape[0]
        dev = tok.device
        t = {"h": torch.empty((self.n_layer + 1, B, self.d_model), dtype=torch.float32, device=dev),
             "q1": torch.empty((self.n_layer, B, self.d_model), dtype=torch.int8, device=dev),
             "q2": torch.empty((self.n_layer, B, self.d_inner), dtype=torch.int8, device=dev),
             "qf": torch.empty((B, self.d_model), dtype=torch.int8, device=dev),
             "logits": torch.empty((B, self.vocab), dtype=torch.float32, device=dev)}
        if want_acc:
            t["acc1"] = torch.empty((self.n_layer, B, self.d_in_proj), dtype=torch.int32, device=dev)
            t["acc2"] = torch.empty((self.n_layer, B, self.d_model), dtype=torch.int32, device=dev)
        call("dfssm_trace_step", self._h, _dp(tok), B, _dp(t["h"]), _dp(t["q1"]), _dp(t["q2"]), _dp(t["qf"]),
             _dp(t["logits"]), _dp(t.get("acc1")), _dp(t.get("acc2")), _stream(stream))
        return t

    def trace_prefill(self, tok, want_acc: bool = False, stream=None):
        """Prefill of tok ([B][T] int32, one chunk) on the batched path, recording, per token row
        m = b * T + t, the residual stream per layer, every int8 activation code and (with
        want_acc) the exact int32 scaffold sums.

        Returns dict(h=[L+1][B*T][d_model], q1=[L][B*T][d_model], q2=[L][B*T][d_inner],
        qf=[B][d_model], logits=[B][vocab]) (the last two for the last position), plus
        acc1=[L][B*T][d_in_proj] and acc2=[L][B*T][d_model] with want_acc."""
        torch = _torch()
        self._check_tok(tok, 2)
        B, T = tok.shape
        M = B * T
        dev = tok.device
        t = {"h": torch.empty((self.n_layer + 1, M, self.d_model), dtype=torch.float32, device=dev),
             "q1": torch.empty((self.n_layer, M, self.d_model), dtype=torch.int8, device=dev),
             "q2": torch.empty((self.n_layer, M, self.d_inner), dtype=torch.int8, device=dev),
             "qf": torch.empty((B, self.d_model), dtype=torch.int8, device=dev),
             "logits": torch.empty((B, self.vocab), dtype=torch.float32, device=dev)}
        if want_acc:
            t["acc1"] = torch.empty((self.n_layer, M, self.d_in_proj), dtype=torch.int32, device=dev)
            t["acc2"] = torch.empty((self.n_layer, M, self.d_model), dtype=torch.int32, device=dev)
        call("dfssm_trace_prefill", self._h, _dp(tok), B, T, _dp(t["h"]), _dp(t["q1"]), _dp(t["q2"]),
             _dp(t["qf"]), _dp(t["logits"]), _dp(t.get("acc1")), _dp(t.get("acc2")), _stream(stream))
        return t

    PATHS = {"auto": 0, "kernels": 1, "persistent": 2, "gemm": 3}

    def set_path(self, path: str) -> None:
        """Execution path: "auto", "kernels" (per-layer GEMV kernels), "persistent" (batch 1 required
        on the persistent kernel) or "gemm" (every decode and prefill on the batched GEMM path)."""
        call("dfssm_set_path", self._h, self.PATHS[path])

    KERNELS = {"in_proj": 0, "ssm": 1, "out_proj": 2, "lm_head": 3, "norm_quant": 4,
               "b_rows_in": 5, "b_in_proj": 6, "b_scan": 7, "b_rows_out": 8, "b_out_proj": 9, "b_lm_head": 10}

    def time_kernel(self, kernel: str, batch: int = 1, iters: int = 480, stream=None) -> float:
        """Mean microseconds per launch of one decode-step kernel (leaves the state undefined)."""
        avg = ctypes.c_float()
        call("dfssm_time_kernel", self._h, self.KERNELS[kernel], batch, iters, ctypes.byref(avg), _stream(stream))
        return avg.value

    def profile_persistent(self, tok, n_tokens: int, prof_tokens: int, stream=None):
        """Phase timestamps of the persistent kernel: uint64 [prof_tokens][n_layer+1][grid][10] (100 MHz)."""
        torch = _torch()
        self._check_tok(tok, 1)
        grid = self.n_heads * (self.headdim // 16)
        prof = torch.zeros((prof_tokens, self.n_layer + 1, grid, 10), dtype=torch.int64, device=tok.device)
        call("dfssm_profile_persistent", self._h, _dp(tok), n_tokens, _dp(prof), prof_tokens, _stream(stream))
        return prof

    # -- density-field state codec ---------------------------------------------
    def state_pack(self, seq0: int = 0, nseq: int = 1, stream=None):
        """Density fields of the SSM state of slots [seq0, seq0 + nseq): (field uint32
        [nseq][L][H][P][d_state/8], scale fp32 [nseq][L][H][P]) on the device."""
        torch = _torch()
        dev = torch.device("cuda", self.device)
        field = torch.empty((nseq, self.n_layer, self.n_heads, self.headdim, self.d_state // 8), dtype=torch.int32,
                            device=dev)
        scale = torch.empty((nseq, self.n_layer, self.n_heads, self.headdim), dtype=torch.float32, device=dev)
        call("dfssm_state_pack", self._h, seq0, nseq, _dp(field), _dp(scale), _stream(stream))
        return field, scale

    def state_unpack(self, field, scale, seq0: int = 0, stream=None) -> None:
        """Replace the SSM state of slots [seq0, seq0 + nseq) by the fields' readout."""
        nseq = field.shape[0]
        call("dfssm_state_unpack", self._h, seq0, nseq, _dp(field), _dp(scale), _stream(stream))

    def state_roundtrip(self, seq0: int = 0, nseq: int = 1, stream=None) -> None:
        """Pass the SSM state of slots [seq0, seq0 + nseq) through the density codec in place."""
        call("dfssm_state_roundtrip", self._h, seq0, nseq, _stream(stream))

    def check(self, stream=None) -> None:
        call("dfssm_check_device", self._h, _stream(stream))

    def device_bytes(self) -> int:
        n = ctypes.c_size_t()
        call("dfssm_device_bytes", self._h, ctypes.byref(n))
        return n.value


def k_quant(u, stream=None):
    """Per-row int8 quantiser on the GPU: u fp32 [rows][n] -> (q int8, s fp32 [rows])."""
    torch = _torch()
    rows, n = u.shape
    q = torch.empty((rows, n), dtype=torch.int8, device=u.device)
    s = torch.empty((rows,), dtype=torch.float32, device=u.device)
    call("dfssm_k_quant", _dp(u), rows, n, _dp(q), _dp(s), _stream(stream))
    return q, s


def k_density_encode(x, stream=None):
    """Density fields of fp32 rows x [rows][n] (n in 16, 32, 64, 128): (field int32 [rows][n/8], scale [rows])."""
    torch = _torch()
    rows, n = x.shape
    field = torch.empty((rows, n // 8), dtype=torch.int32, device=x.device)
    scale = torch.empty((rows,), dtype=torch.float32, device=x.device)
    call("dfssm_k_density_encode", _dp(x), rows, n, _dp(field), _dp(scale), _stream(stream))
    return field, scale


def k_density_decode(field, scale, stream=None):
    """Popcount readout of density fields: fp32 [rows][n]."""
    torch = _torch()
    rows, w = field.shape
    n = 8 * w
    x = torch.empty((rows, n), dtype=torch.float32, device=field.device)
    call("dfssm_k_density_decode", _dp(field), _dp(scale), rows, n, _dp(x), _stream(stream))
    return x


def k_gemm(bits, sw, A, sA, Bm, sB, q, s, stream=None):
    """The same projection on the batched path's int8 matrix-core GEMM (rank 16)."""
    torch = _torch()
    d_out = bits.shape[0]
    d_in = bits.shape[1] * 32
    M = q.shape[0]
    acc = torch.empty((M, d_out), dtype=torch.int32, device=q.device)
    y = torch.empty((M, d_out), dtype=torch.float32, device=q.device)
    call("dfssm_k_gemm", _dp(bits), _dp(sw), _dp(A), _dp(sA), _dp(Bm), _dp(sB), d_in, d_out, _dp(q), _dp(s), M,
         _dp(acc), _dp(y), _stream(stream))
    return acc, y


def k_gemm_noalloc(bits, sw, A, sA, Bm, sB, q, s, acc=None, y=None, stream=None):
    """k_gemm without any device allocation by the library (static per-GPU scratch; outputs may be
    passed in so the call allocates nothing at all)."""
    torch = _torch()
    d_out = bits.shape[0]
    d_in = bits.shape[1] * 32
    M = q.shape[0]
    if acc is None:
        acc = torch.empty((M, d_out), dtype=torch.int32, device=q.device)
    if y is None:
        y = torch.empty((M, d_out), dtype=torch.float32, device=q.device)
    call("dfssm_k_gemm_noalloc", _dp(bits), _dp(sw), _dp(A), _dp(sA), _dp(Bm), _dp(sB), d_in, d_out, _dp(q), _dp(s),
         M, _dp(acc), _dp(y), _stream(stream))
    return acc, y


def k_proj(bits, sw, A, sA, Bm, sB, q, s, stream=None):
    """Scaffold + LoRA projection of int8 rows q [B][d_in] -> (acc int32, y fp32) [B][d_out]."""
    torch = _torch()
    d_out = bits.shape[0]
    d_in = bits.shape[1] * 32
    r = A.shape[0]
    B = q.shape[0]
    acc = torch.empty((B, d_out), dtype=torch.int32, device=q.device)
    y = torch.empty((B, d_out), dtype=torch.float32, device=q.device)
    call("dfssm_k_proj", _dp(bits), _dp(sw), _dp(A), _dp(sA), _dp(Bm), _dp(sB), d_in, d_out, r, _dp(q), _dp(s), B,
         _dp(acc), _dp(y), _stream(stream))
    return acc, y
