"""Python face of the CPU oracle (ctypes over oracle/liboracle.so).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It never imports the
GPU package and the GPU package never imports it; the two share only the
seeded input generator in ``synth``.

Every function mirrors one function of ``dfssm_oracle.c`` (see that file's
header for what is computed, which passage of the pages each step follows,
and the readings taken where the pages are silent).  All floating-point
results are fp64.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from synth import LAYER_KINDS, GLOBAL_KINDS, Shape

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.or_quant_f32.argtypes = [_p, _i, _p, _p]
        L.or_quant.argtypes = [_p, _i, _p, _p]
        L.or_rmsnorm.argtypes = [_p, _p, _i, _p]
        L.or_scaffold_acc.argtypes = [_p, _i, _i, _p, _p]
        L.or_scaffold_acc.restype = _i
        L.or_proj.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _p, ctypes.c_float, _p, _p, _p]
        L.or_proj.restype = _i
        L.or_unpack_signs.argtypes = [_p, _i, _i, _p]
        L.or_sign_acc.argtypes = [_p, _i, _i, _p, _p]
        L.or_sign_acc.restype = _i
        L.or_conv_step.argtypes = [_p, _p, _p, _i, _i, _p, _p]
        L.or_ssm_step.argtypes = [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p]
        L.or_gated_rmsnorm.argtypes = [_p, _p, _p, _i, _p]
        L.or_layer_step.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]
        L.or_layer_step.restype = _i
        L.or_quant_forced.argtypes = [_p, _i, _p, ctypes.c_double, _p, _p, _p]
        L.or_quant_forced.restype = _i
        L.or_layer_step_forced.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_double,
                                           _p, _p]
        L.or_layer_step_forced.restype = _i
        L.or_lm_head_forced.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_double, _p, _p]
        L.or_lm_head_forced.restype = _i
        L.or_lm_head.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p]
        L.or_lm_head.restype = _i
        L.or_embed.argtypes = [_p, _p, _p, _i, _p]
        L.or_decode_step.argtypes = [_p, _p, _p, _p, _i, _p, _p]
        L.or_decode_step.restype = _i
        L.or_prefill.argtypes = [_p, _p, _p, _p, _p, _i, _p]
        L.or_prefill.restype = _i
        L.or_num_threads.restype = _i
        L.or_density_encode.argtypes = [_p, _i, _p, _p]
        L.or_density_decode.argtypes = [_p, ctypes.c_float, _i, _p]
        _lib = L
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(lib().or_num_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _shape_arr(s: Shape) -> np.ndarray:
    return np.array(s.as_ints(), dtype=np.int32)


# ---------------------------------------------------------------------------
# stage functions
# ---------------------------------------------------------------------------


def quant_f32(u) -> Tuple[np.ndarray, np.float32]:
    u = _c(u, np.float32)
    q = np.empty(u.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().or_quant_f32(_ptr(u), u.size, _ptr(q), _ptr(s))
    return q, s[0]


def quant(u) -> Tuple[np.ndarray, np.float32]:
    u = _c(u, np.float64)
    q = np.empty(u.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().or_quant(_ptr(u), u.size, _ptr(q), _ptr(s))
    return q, s[0]


# Half-width, in units of the int8 step, of the band around a rounding tie in
# which a code one away from the oracle's own is still a correct result.  An
# fp32 implementation's scaled value u * 127 / amax differs from the oracle's
# by its accumulated rounding error: a few ulp of u after the residual stream
# has gone through the stack (relative 1e-6 at most), times |u * 127/amax|
# <= 127, i.e. below 1.3e-4; the band keeps a margin of about 8x over that.
TIE_BAND = 1e-3


def quant_forced(u, force, delta: float = TIE_BAND) -> Tuple[np.ndarray, np.float32, int, int]:
    """Quantise u (fp64) taking the proposed codes where they are valid roundings.

    Returns (q, s, number of rejected proposals, number of accepted proposals
    that differ from the oracle's own code)."""
    u = _c(u, np.float64)
    force = _c(force, np.int8)
    assert force.size == u.size
    q = np.empty(u.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    fl = np.zeros(1, dtype=np.int32)
    bad = lib().or_quant_forced(_ptr(u), u.size, _ptr(force), float(delta), _ptr(q), _ptr(s), _ptr(fl))
    return q, s[0], bad, int(fl[0])


def density_encode(x) -> Tuple[np.ndarray, np.float32]:
    """Density field of one state row x (fp32 [n]): (field uint32 [ceil(4n/32)], scale fp32)."""
    x = _c(x, np.float32)
    n = x.size
    field = np.zeros((4 * n + 31) // 32, dtype=np.uint32)
    sc = np.zeros(1, dtype=np.float32)
    lib().or_density_encode(_ptr(x), n, _ptr(field), _ptr(sc))
    return field, sc[0]


def density_decode(field, scale, n: int) -> np.ndarray:
    """Popcount readout of a density field: fp32 [n]."""
    field = _c(field, np.uint32)
    assert field.size == (4 * n + 31) // 32
    x = np.empty(n, dtype=np.float32)
    lib().or_density_decode(_ptr(field), float(np.float32(scale)), n, _ptr(x))
    return x


def density_roundtrip_state(ssm) -> np.ndarray:
    """decode(encode(row)) of every d_state row of an SSM state [..., d_state], in fp32 (returned as fp64)."""
    a = np.asarray(ssm, dtype=np.float64)
    rows = a.reshape(-1, a.shape[-1]).astype(np.float32)
    out = np.empty_like(rows)
    for r in range(rows.shape[0]):
        f, sc = density_encode(rows[r])
        out[r] = density_decode(f, sc, rows.shape[1])
    return out.reshape(a.shape).astype(np.float64)


def rmsnorm(x, w) -> np.ndarray:
    x = _c(x, np.float64)
    w = _c(w, np.float32)
    u = np.empty_like(x)
    lib().or_rmsnorm(_ptr(x), _ptr(w), x.size, _ptr(u))
    return u


def scaffold_acc(bits, q) -> np.ndarray:
    bits = _c(bits, np.uint32)
    q = _c(q, np.int8)
    d_out, words = bits.shape
    assert words * 32 == q.size
    acc = np.empty(d_out, dtype=np.int32)
    rc = lib().or_scaffold_acc(_ptr(bits), d_out, q.size, _ptr(q), _ptr(acc))
    if rc != 0:
        raise OverflowError("scaffold accumulator exceeds int32")
    return acc


def unpack_signs(bits, d_in: int) -> np.ndarray:
    """The scaffold as a dense int8 sign matrix [d_out][d_in] (+1 where the bit is set)."""
    bits = _c(bits, np.uint32)
    d_out = bits.shape[0]
    assert bits.size == d_out * (d_in // 32)
    out = np.empty((d_out, d_in), dtype=np.int8)
    lib().or_unpack_signs(_ptr(bits), d_out, d_in, _ptr(out))
    return out


def sign_acc(signs, q) -> np.ndarray:
    """Scaffold sums from an unpacked sign matrix (the same integers as scaffold_acc)."""
    signs = _c(signs, np.int8)
    q = _c(q, np.int8)
    d_out, d_in = signs.shape
    acc = np.empty(d_out, dtype=np.int32)
    if lib().or_sign_acc(_ptr(signs), d_out, d_in, _ptr(q), _ptr(acc)) != 0:
        raise OverflowError("d_in too large for int32 row sums")
    return acc


def proj(bits, sw, A, sA, B, sB, q, s) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Scaffold + LoRA projection. Returns (y fp64, acc int32, ta int64)."""
    bits = _c(bits, np.uint32)
    d_out, words = bits.shape
    d_in = words * 32
    A = _c(A, np.int8)
    B = _c(B, np.int8)
    r = A.shape[0]
    assert A.shape == (r, d_in) and B.shape == (d_out, r)
    sw, sA, sB = _c(sw, np.float32), _c(sA, np.float32), _c(sB, np.float32)
    q = _c(q, np.int8)
    y = np.empty(d_out, dtype=np.float64)
    acc = np.empty(d_out, dtype=np.int32)
    ta = np.empty(r, dtype=np.int64)
    rc = lib().or_proj(_ptr(bits), _ptr(sw), _ptr(A), _ptr(sA), _ptr(B), _ptr(sB), d_in, d_out, r,
                       _ptr(q), float(s), _ptr(y), _ptr(acc), _ptr(ta))
    if rc != 0:
        raise OverflowError("scaffold accumulator exceeds int32")
    return y, acc, ta


def conv_step(xin, w, b, state) -> np.ndarray:
    """One conv shift-register step; `state` ([C][K-1], fp64) is updated in place."""
    xin = _c(xin, np.float64)
    w = _c(w, np.float32)
    b = _c(b, np.float32)
    C, K = w.shape
    assert state.dtype == np.float64 and state.shape == (C, K - 1) and state.flags.c_contiguous
    out = np.empty(C, dtype=np.float64)
    lib().or_conv_step(_ptr(xin), _ptr(w), _ptr(b), C, K, _ptr(state), _ptr(out))
    return out


def ssm_step(x, Bv, Cv, dt_raw, A_log, dt_bias, D, S) -> Tuple[np.ndarray, np.ndarray]:
    """One SSM step; `S` ([H][P][N], fp64) is updated in place. Returns (y [H*P], dt [H])."""
    H, P, N = S.shape
    assert S.dtype == np.float64 and S.flags.c_contiguous
    x = _c(x, np.float64).reshape(-1)
    Bv, Cv, dt_raw = _c(Bv, np.float64), _c(Cv, np.float64), _c(dt_raw, np.float64)
    A_log, dt_bias, D = _c(A_log, np.float32), _c(dt_bias, np.float32), _c(D, np.float32)
    y = np.empty(H * P, dtype=np.float64)
    dt = np.empty(H, dtype=np.float64)
    lib().or_ssm_step(_ptr(x), _ptr(Bv), _ptr(Cv), _ptr(dt_raw), _ptr(A_log), _ptr(dt_bias), _ptr(D),
                      H, P, N, _ptr(S), _ptr(y), _ptr(dt))
    return y, dt


def gated_rmsnorm(y, z, w) -> np.ndarray:
    y, z, w = _c(y, np.float64), _c(z, np.float64), _c(w, np.float32)
    u = np.empty_like(y)
    lib().or_gated_rmsnorm(_ptr(y), _ptr(z), _ptr(w), y.size, _ptr(u))
    return u


# ---------------------------------------------------------------------------
# layer / model
# ---------------------------------------------------------------------------


# A layer's pointer array: the 19 tensors in LAYER_KINDS order, then the
# optional unpacked sign matrices of the two scaffolds (None -> the oracle
# reads the bits).
SIGN_KINDS = ["in_signs", "out_signs"]
LW_STRIDE = len(LAYER_KINDS) + len(SIGN_KINDS)


def with_signs(s: Shape, layer: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """A copy of a layer's weights with its scaffolds also unpacked to sign matrices."""
    d = dict(layer)
    d["in_signs"] = unpack_signs(layer["in_bits"], s.d_model)
    d["out_signs"] = unpack_signs(layer["out_bits"], s.d_inner)
    return d


def _fill_layer_ptrs(arr, base: int, layer: Dict[str, np.ndarray], keep: List[np.ndarray]) -> None:
    for j, k in enumerate(LAYER_KINDS + SIGN_KINDS):
        if layer.get(k) is None:
            arr[base + j] = None
            continue
        a = np.ascontiguousarray(layer[k])
        keep.append(a)
        arr[base + j] = a.ctypes.data


def _layer_ptr_array(layer: Dict[str, np.ndarray], keep: List[np.ndarray]):
    arr = (ctypes.c_void_p * LW_STRIDE)()
    _fill_layer_ptrs(arr, 0, layer, keep)
    return arr


def dbg_layout(s: Shape) -> Dict[str, Tuple[int, int]]:
    sizes = [("zxbcdt", s.d_in_proj), ("xc", s.conv_dim), ("dt", s.n_heads), ("y", s.d_inner),
             ("u2", s.d_inner), ("out", s.d_model)]
    off, lay = 0, {}
    for name, n in sizes:
        lay[name] = (off, off + n)
        off += n
    lay["_total"] = (0, off)
    return lay


class State:
    """Per-sequence recurrent state of a whole stack (fp64)."""

    def __init__(self, s: Shape):
        self.conv = np.zeros((s.n_layer, s.conv_dim, s.d_conv - 1), dtype=np.float64)
        self.ssm = np.zeros((s.n_layer, s.n_heads, s.headdim, s.d_state), dtype=np.float64)

    def copy(self) -> "State":
        c = State.__new__(State)
        c.conv = self.conv.copy()
        c.ssm = self.ssm.copy()
        return c


class ForcedCodeError(AssertionError):
    """A proposed int8 code is not a correct rounding of the oracle's value."""


def _count(stats: Optional[Dict[str, int]], flips: int, codes: int) -> None:
    if stats is not None:
        stats["flips"] = stats.get("flips", 0) + int(flips)
        stats["codes"] = stats.get("codes", 0) + int(codes)


def layer_step(s: Shape, layer: Dict[str, np.ndarray], h_in, conv_state: np.ndarray, ssm_state: np.ndarray,
               want_dbg: bool = False, q1_force=None, q2_force=None, delta: float = TIE_BAND,
               stats: Optional[Dict[str, int]] = None):
    """One layer, one token. conv_state [conv_dim][K-1] and ssm_state [H][P][N] (fp64) update in place.

    q1_force / q2_force (optional int8 codes) are taken where they are correct
    roundings (see quant_forced); any other proposal raises ForcedCodeError.
    stats (optional dict) accumulates "flips", the proposed codes taken that
    differ from the oracle's own, and "codes", the proposed codes seen.
    Returns h_out, or (h_out, dbg dict) with the intermediate vectors and the
    int8 activations (q1, s1, q2, s2) when want_dbg is set.
    """
    keep: List[np.ndarray] = []
    lw = _layer_ptr_array(layer, keep)
    h_in = _c(h_in, np.float64)
    assert conv_state.dtype == np.float64 and conv_state.flags.c_contiguous
    assert ssm_state.dtype == np.float64 and ssm_state.flags.c_contiguous
    assert conv_state.shape == (s.conv_dim, s.d_conv - 1)
    assert ssm_state.shape == (s.n_heads, s.headdim, s.d_state)
    h_out = np.empty(s.d_model, dtype=np.float64)
    lay = dbg_layout(s)
    dbg = np.empty(lay["_total"][1], dtype=np.float64) if want_dbg else None
    q1 = np.empty(s.d_model, dtype=np.int8) if want_dbg else None
    q2 = np.empty(s.d_inner, dtype=np.int8) if want_dbg else None
    s1 = np.zeros(1, dtype=np.float32)
    s2 = np.zeros(1, dtype=np.float32)
    sh = _shape_arr(s)
    f1 = None if q1_force is None else _c(q1_force, np.int8)
    f2 = None if q2_force is None else _c(q2_force, np.int8)
    if f1 is not None:
        assert f1.size == s.d_model
    if f2 is not None:
        assert f2.size == s.d_inner
    rej = np.zeros(1, dtype=np.int32)
    fl = np.zeros(1, dtype=np.int32)
    rc = lib().or_layer_step_forced(_ptr(sh), lw, _ptr(h_in), _ptr(conv_state), _ptr(ssm_state), _ptr(h_out),
                                    _ptr(dbg), _ptr(q1), _ptr(s1), _ptr(q2), _ptr(s2), _ptr(f1), _ptr(f2),
                                    float(delta), _ptr(rej), _ptr(fl))
    if rc != 0:
        raise OverflowError("integer accumulator overflow")
    if rej[0]:
        raise ForcedCodeError(f"{int(rej[0])} proposed int8 codes are not correct roundings")
    _count(stats, fl[0], (0 if f1 is None else f1.size) + (0 if f2 is None else f2.size))
    if not want_dbg:
        return h_out
    d = {k: dbg[a:b].copy() for k, (a, b) in lay.items() if k != "_total"}
    d.update(q1=q1, s1=s1[0], q2=q2, s2=s2[0])
    return h_out, d


class Model:
    """A whole stack's weights held for the oracle (canonical layouts).

    With signs (the default) each layer's scaffolds are also held unpacked as
    int8 sign matrices, which the oracle then reads instead of the bits (the
    same integer sums, several times faster); self.weights["layers"] are those
    layer dicts, for oracle.layer_step."""

    def __init__(self, s: Shape, weights: Dict[str, object], signs: bool = True):
        self.s = s
        self._keep: List[np.ndarray] = []
        layers = [with_signs(s, lay) if signs else dict(lay) for lay in weights["layers"]]
        weights = dict(weights, layers=layers)
        n = s.n_layer * LW_STRIDE + len(GLOBAL_KINDS)
        self._ptrs = (ctypes.c_void_p * n)()
        for l in range(s.n_layer):
            _fill_layer_ptrs(self._ptrs, l * LW_STRIDE, layers[l], self._keep)
        j = s.n_layer * LW_STRIDE
        for k in GLOBAL_KINDS:
            a = np.ascontiguousarray(weights[k])
            self._keep.append(a)
            self._ptrs[j] = a.ctypes.data
            j += 1
        self._sh = _shape_arr(s)
        self.weights = weights

    def decode_step(self, st: State, tok: int, want_logits: bool = True, want_trace: bool = False):
        """Returns (next_token, logits or None, h_trace or None)."""
        s = self.s
        logits = np.empty(s.vocab, dtype=np.float64) if want_logits else None
        trace = np.empty((s.n_layer + 1, s.d_model), dtype=np.float64) if want_trace else None
        nxt = lib().or_decode_step(_ptr(self._sh), self._ptrs, _ptr(st.conv), _ptr(st.ssm), int(tok),
                                   _ptr(logits), _ptr(trace))
        if nxt == -2:
            raise ValueError("token out of range or accumulator overflow")
        return nxt, logits, trace

    def prefill(self, st: State, toks: Sequence[int], want_logits: bool = True):
        toks = np.ascontiguousarray(toks, dtype=np.int32)
        s = self.s
        logits = np.empty(s.vocab, dtype=np.float64) if want_logits else None
        nxt = lib().or_prefill(_ptr(self._sh), self._ptrs, _ptr(st.conv), _ptr(st.ssm), _ptr(toks),
                               int(toks.size), _ptr(logits))
        if nxt == -2:
            raise ValueError("token out of range or accumulator overflow")
        return nxt, logits

    def lm_head(self, h, qf_force=None, delta: float = TIE_BAND, stats: Optional[Dict[str, int]] = None):
        """Final norm + tied int8 LM head. Returns (argmax, logits, qf, sf).

        qf_force and stats as for layer_step."""
        s = self.s
        h = _c(h, np.float64)
        logits = np.empty(s.vocab, dtype=np.float64)
        qf = np.empty(s.d_model, dtype=np.int8)
        sf = np.zeros(1, dtype=np.float32)
        E = self.weights["E"]
        sE = self.weights["sE"]
        fn = self.weights["final_norm"]
        ff = None if qf_force is None else _c(qf_force, np.int8)
        rej = np.zeros(1, dtype=np.int32)
        fl = np.zeros(1, dtype=np.int32)
        best = lib().or_lm_head_forced(_ptr(self._sh), _ptr(np.ascontiguousarray(E)), _ptr(np.ascontiguousarray(sE)),
                                       _ptr(np.ascontiguousarray(fn)), _ptr(h), _ptr(logits), _ptr(qf), _ptr(sf),
                                       _ptr(ff), float(delta), _ptr(rej), _ptr(fl))
        if rej[0]:
            raise ForcedCodeError(f"{int(rej[0])} proposed int8 codes are not correct roundings")
        _count(stats, fl[0], 0 if ff is None else ff.size)
        return best, logits, qf, sf[0]

    def embed(self, tok: int) -> np.ndarray:
        s = self.s
        h = np.empty(s.d_model, dtype=np.float64)
        lib().or_embed(_ptr(self._sh), _ptr(np.ascontiguousarray(self.weights["E"])),
                       _ptr(np.ascontiguousarray(self.weights["sE"])), int(tok), _ptr(h))
        return h
