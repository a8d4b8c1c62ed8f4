"""Seeded synthetic inputs for the DF-SSM decode path.

This module is the one piece shared by the CPU oracle's tests and the GPU
path's harness.  It holds only random-number generation and the shapes of the
workloads; none of the model's arithmetic (no quantisation, no projections, no
recurrence) lives here.

Generator
---------
Every value is a pure function of (seed, tid, index), so any element can be
drawn on its own and the device library can draw the same numbers without
sharing code with this file.

* ``mix(x)``: the SplitMix64 output function (Steele, Lea & Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014): add the golden
  gamma 0x9E3779B97F4A7C15, then two xor-shift-multiply rounds and a final
  xor-shift.  ``mix`` applied to successive multiples of the gamma is the
  sequence of the published ``splitmix64`` generator.
* ``draw(seed, tid, i) = mix(mix(seed ^ (tid << 32)) + i)`` (mod 2**64), with
  ``i`` the element's row-major index in the tensor's canonical layout.
* uniform ``u = (draw >> 40) * 2**-24`` in [0, 1) (24 bits, exact in fp32).
* ``U(a, b) = fp32(a + (b - a) * u)``: fp64 multiply, fp64 add (no fused
  multiply-add), one round-to-nearest-even to fp32.
* int8 ``U[-127, 127] = (draw % 255) - 127``.
* packed sign words: ``word = draw >> 32``; bit ``k`` of word ``j`` of row
  ``o`` is the sign of weight ``(o, 32 j + k)``, so every weight is an
  independent fair coin.
* "N(0, 1)": Irwin-Hall, ``sum_{k<12} u(seed, tid, 12 i + k) - 6`` summed in
  fp64 (exact: 24-bit terms), rounded once to fp32.
* token ids: ``draw % vocab``.

Tensor ids: per layer ``tid = 64 * layer + kind`` with kinds in ``LAYER_KINDS``
order; the embedding, its scale and the final norm use 4096, 4097, 4098;
token and activation streams use ``8192 + stream``.

Distributions (scaffold, LoRA, A_log, dt_bias, D as the tiny 2-layer workload
states them; the others are this project's choice, chosen so that an index
mistake changes results): scaffold signs fair coins; scaffold row scales
U(0.01, 0.05); LoRA A and B int8 U[-127, 127] with constant row scales 1e-3;
A_log U(0, ln 16); dt_bias U(-4, -1); D "N(0,1)"; conv weight and bias
U(-0.5, 0.5); RMSNorm weights U(0.5, 1.5); embedding int8 U[-127, 127] with
row scales U(0.01, 0.02).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterator, List, Tuple

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_U64 = np.uint64

LN16 = 2.772588722239781  # ln(16) as the fp64 constant used for the A_log upper bound

# ---------------------------------------------------------------------------
# shapes
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Shape:
    """Dimensions of a DF-SSM Mamba-2 stack (ngroups = 1)."""

    n_layer: int
    d_model: int
    d_inner: int
    d_state: int
    headdim: int
    vocab: int
    d_conv: int = 4
    rank: int = 16

    @property
    def n_heads(self) -> int:
        return self.d_inner // self.headdim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.d_state

    @property
    def d_in_proj(self) -> int:
        return 2 * self.d_inner + 2 * self.d_state + self.n_heads

    def as_ints(self) -> List[int]:
        return [self.n_layer, self.d_model, self.d_inner, self.d_state, self.headdim,
                self.vocab, self.d_conv, self.rank]


# The five workloads: the tiny 2-layer stack; one 1.3B-shaped layer; the full
# 48-layer 1.3B-shaped model (batch-1 decode, batch-32 decode, 8 x 2048 prefill).
TINY = Shape(n_layer=2, d_model=256, d_inner=512, d_state=16, headdim=32, vocab=1024)
LAYER_1P3B = Shape(n_layer=1, d_model=2048, d_inner=4096, d_state=128, headdim=64, vocab=256)
FULL_1P3B = Shape(n_layer=48, d_model=2048, d_inner=4096, d_state=128, headdim=64, vocab=50288)

SEED_BASE = 0xDF55  # workload k uses seed SEED_BASE + k


# kind -> (name, shape function, dtype, distribution)
LAYER_KINDS: List[str] = [
    "in_bits", "in_sw", "in_A", "in_sA", "in_B", "in_sB",
    "out_bits", "out_sw", "out_A", "out_sA", "out_B", "out_sB",
    "conv_w", "conv_b", "A_log", "dt_bias", "D", "norm_w", "gnorm_w",
]
GLOBAL_KINDS: List[str] = ["E", "sE", "final_norm"]
GLOBAL_TID = {"E": 4096, "sE": 4097, "final_norm": 4098}
STREAM_TID = 8192


def layer_tensor_spec(s: Shape, kind: str) -> Tuple[Tuple[int, ...], np.dtype]:
    r = s.rank
    spec = {
        "in_bits": ((s.d_in_proj, s.d_model // 32), np.uint32),
        "in_sw": ((s.d_in_proj,), np.float32),
        "in_A": ((r, s.d_model), np.int8),
        "in_sA": ((r,), np.float32),
        "in_B": ((s.d_in_proj, r), np.int8),
        "in_sB": ((s.d_in_proj,), np.float32),
        "out_bits": ((s.d_model, s.d_inner // 32), np.uint32),
        "out_sw": ((s.d_model,), np.float32),
        "out_A": ((r, s.d_inner), np.int8),
        "out_sA": ((r,), np.float32),
        "out_B": ((s.d_model, r), np.int8),
        "out_sB": ((s.d_model,), np.float32),
        "conv_w": ((s.conv_dim, s.d_conv), np.float32),
        "conv_b": ((s.conv_dim,), np.float32),
        "A_log": ((s.n_heads,), np.float32),
        "dt_bias": ((s.n_heads,), np.float32),
        "D": ((s.n_heads,), np.float32),
        "norm_w": ((s.d_model,), np.float32),
        "gnorm_w": ((s.d_inner,), np.float32),
    }
    shp, dt = spec[kind]
    return shp, np.dtype(dt)


def global_tensor_spec(s: Shape, kind: str) -> Tuple[Tuple[int, ...], np.dtype]:
    spec = {
        "E": ((s.vocab, s.d_model), np.int8),
        "sE": ((s.vocab,), np.float32),
        "final_norm": ((s.d_model,), np.float32),
    }
    shp, dt = spec[kind]
    return shp, np.dtype(dt)


# ---------------------------------------------------------------------------
# counter-based generator
# ---------------------------------------------------------------------------


def mix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrap-around arithmetic)."""
    x = np.asarray(x, dtype=_U64)
    with np.errstate(over="ignore"):
        z = x + _U64(GAMMA)
        z = (z ^ (z >> _U64(30))) * _U64(_M1)
        z = (z ^ (z >> _U64(27))) * _U64(_M2)
        return z ^ (z >> _U64(31))


def mix64_int(x: int) -> int:
    """Scalar SplitMix64 output function on a Python int."""
    m = (1 << 64) - 1
    z = (x + GAMMA) & m
    z = ((z ^ (z >> 30)) * _M1) & m
    z = ((z ^ (z >> 27)) * _M2) & m
    return z ^ (z >> 31)


def stream_key(seed: int, tid: int) -> int:
    m = (1 << 64) - 1
    return mix64_int((seed ^ ((tid << 32) & m)) & m)


def draws(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    """draw(seed, tid, i) for i in [start, start + count)."""
    key = _U64(stream_key(seed, tid))
    idx = np.arange(start, start + count, dtype=_U64)
    with np.errstate(over="ignore"):
        return mix64(idx + key)


_CHUNK = 1 << 22


def _chunked(n: int) -> Iterator[Tuple[int, int]]:
    for b in range(0, n, _CHUNK):
        yield b, min(n, b + _CHUNK)


def uniform01(d: np.ndarray) -> np.ndarray:
    return (d >> _U64(40)).astype(np.float64) * (2.0 ** -24)


def gen_uniform(seed: int, tid: int, n: int, a: float, b: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for lo, hi in _chunked(n):
        u = uniform01(draws(seed, tid, lo, hi - lo))
        out[lo:hi] = (np.float64(a) + (np.float64(b) - np.float64(a)) * u).astype(np.float32)
    return out


def gen_int8(seed: int, tid: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int8)
    for lo, hi in _chunked(n):
        d = draws(seed, tid, lo, hi - lo)
        out[lo:hi] = ((d % _U64(255)).astype(np.int64) - 127).astype(np.int8)
    return out


def gen_words(seed: int, tid: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    for lo, hi in _chunked(n):
        out[lo:hi] = (draws(seed, tid, lo, hi - lo) >> _U64(32)).astype(np.uint32)
    return out


def gen_normal(seed: int, tid: int, n: int, start: int = 0) -> np.ndarray:
    """Irwin-Hall "N(0,1)" values with element indices [start, start + n)."""
    out = np.empty(n, dtype=np.float32)
    step = max(1, _CHUNK // 12)
    for lo in range(0, n, step):
        hi = min(n, lo + step)
        u = uniform01(draws(seed, tid, 12 * (start + lo), 12 * (hi - lo))).reshape(hi - lo, 12)
        acc = np.zeros(hi - lo, dtype=np.float64)
        for k in range(12):  # fixed left-to-right order; every partial sum is exact
            acc = acc + u[:, k]
        out[lo:hi] = (acc - 6.0).astype(np.float32)
    return out


def gen_tokens(seed: int, stream: int, n: int, vocab: int, start: int = 0) -> np.ndarray:
    d = draws(seed, STREAM_TID + stream, start, n)
    return (d % _U64(vocab)).astype(np.int32)


def gen_fp16_normal(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """'N(0,1)' activations rounded to fp16 (round-to-nearest-even)."""
    return gen_normal(seed, STREAM_TID + stream, n, start).astype(np.float16)


# ---------------------------------------------------------------------------
# model weights in canonical layout
# ---------------------------------------------------------------------------

_CONST_SCALE = np.float32(1e-3)


def gen_layer_tensor(s: Shape, seed: int, layer: int, kind: str) -> np.ndarray:
    shp, dt = layer_tensor_spec(s, kind)
    n = int(np.prod(shp))
    tid = 64 * layer + LAYER_KINDS.index(kind)
    if kind in ("in_bits", "out_bits"):
        v = gen_words(seed, tid, n)
    elif kind in ("in_sw", "out_sw"):
        v = gen_uniform(seed, tid, n, 0.01, 0.05)
    elif kind in ("in_A", "in_B", "out_A", "out_B"):
        v = gen_int8(seed, tid, n)
    elif kind in ("in_sA", "in_sB", "out_sA", "out_sB"):
        v = np.full(n, _CONST_SCALE, dtype=np.float32)
    elif kind in ("conv_w", "conv_b"):
        v = gen_uniform(seed, tid, n, -0.5, 0.5)
    elif kind == "A_log":
        v = gen_uniform(seed, tid, n, 0.0, LN16)
    elif kind == "dt_bias":
        v = gen_uniform(seed, tid, n, -4.0, -1.0)
    elif kind == "D":
        v = gen_normal(seed, tid, n)
    elif kind in ("norm_w", "gnorm_w"):
        v = gen_uniform(seed, tid, n, 0.5, 1.5)
    else:
        raise KeyError(kind)
    return v.astype(dt, copy=False).reshape(shp)


def gen_global_tensor(s: Shape, seed: int, kind: str) -> np.ndarray:
    shp, dt = global_tensor_spec(s, kind)
    n = int(np.prod(shp))
    tid = GLOBAL_TID[kind]
    if kind == "E":
        v = gen_int8(seed, tid, n)
    elif kind == "sE":
        v = gen_uniform(seed, tid, n, 0.01, 0.02)
    elif kind == "final_norm":
        v = gen_uniform(seed, tid, n, 0.5, 1.5)
    else:
        raise KeyError(kind)
    return v.astype(dt, copy=False).reshape(shp)


def gen_layer(s: Shape, seed: int, layer: int) -> Dict[str, np.ndarray]:
    return {k: gen_layer_tensor(s, seed, layer, k) for k in LAYER_KINDS}


def gen_model(s: Shape, seed: int, with_embedding: bool = True) -> Dict[str, object]:
    """All weights of a stack: {"layers": [dict per layer], "E", "sE", "final_norm"}."""
    m: Dict[str, object] = {"layers": [gen_layer(s, seed, l) for l in range(s.n_layer)]}
    if with_embedding:
        for k in GLOBAL_KINDS:
            m[k] = gen_global_tensor(s, seed, k)
    return m


def model_bytes(s: Shape) -> Dict[str, int]:
    """Storage of the encoded model, by component (bytes)."""
    per = {k: int(np.prod(layer_tensor_spec(s, k)[0])) * layer_tensor_spec(s, k)[1].itemsize
           for k in LAYER_KINDS}
    scaffold = s.n_layer * (per["in_bits"] + per["out_bits"])
    lora = s.n_layer * (per["in_A"] + per["in_B"] + per["out_A"] + per["out_B"])
    other_layer = s.n_layer * sum(per[k] for k in LAYER_KINDS
                                  if k not in ("in_bits", "out_bits", "in_A", "in_B", "out_A", "out_B"))
    emb = s.vocab * s.d_model
    other_global = s.vocab * 4 + s.d_model * 4
    return {"scaffold": scaffold, "embedding": emb, "lora": lora,
            "other": other_layer + other_global}
