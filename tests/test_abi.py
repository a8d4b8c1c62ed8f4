"""The C-ABI library loads on a machine without a GPU and exports every
function that include/dfssm.h declares (no compute calls here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dfssm.h")
LIB = os.path.join(ROOT, "bit_quantized_mamba_amd", "libdfssm.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dfssm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dfssm_arena_bytes", "dfssm_create", "dfssm_load_synthetic", "dfssm_decode_step", "dfssm_prefill",
              "dfssm_generate", "dfssm_layer_step", "dfssm_layer_step_f16", "dfssm_trace_step", "dfssm_k_proj",
              "dfssm_k_quant", "dfssm_k_gemm", "dfssm_get_state", "dfssm_set_state", "dfssm_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        pytest.fail("libdfssm.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    from bit_quantized_mamba_amd import _lib
    assert sorted(_lib.EXPORTS) == declared_functions()


def test_version_and_argument_errors_without_gpu():
    from bit_quantized_mamba_amd import _lib
    L = _lib.load()
    assert b"gfx950" in L.dfssm_version()
    # host-side validation fails before any device work
    cfg = _lib.DfssmConfig(1, 100, 512, 16, 32, 10, 4, 16, 1, 1e-5, 0)  # d_model not a multiple of 128
    h = ctypes.c_void_p()
    rc = L.dfssm_create(ctypes.byref(cfg), 0, None, 0, ctypes.byref(h))
    assert rc == -5 and not h.value
    assert b"d_model" in L.dfssm_last_error(None)
    assert L.dfssm_k_quant(None, 1, 1, None, None, None) == -1
    n = ctypes.c_size_t()
    assert L.dfssm_arena_bytes(ctypes.byref(cfg), ctypes.byref(n)) == -5


def test_arena_bytes_host_only():
    # the arena size is host arithmetic: no device is touched
    import synth
    from bit_quantized_mamba_amd import Engine
    s = synth.FULL_1P3B

    def size(max_batch, rows=0):
        return Engine.arena_bytes(s.n_layer, s.d_model, s.d_inner, s.d_state, s.headdim, s.vocab,
                                  max_batch=max_batch, max_chunk_rows=rows)

    one = size(1)
    weights = sum(synth.model_bytes(s).values())
    state_per_seq = 4 * s.n_layer * (s.n_heads * s.headdim * s.d_state + (s.d_conv - 1) * s.conv_dim)
    assert one > weights + state_per_seq
    # one more sequence slot costs at least its recurrent state
    assert size(2) - one >= state_per_seq
    # the batched-path workspace grows with the chunk rows (fp32 h, in_proj output, conv output, g per row)
    per_row = 4 * (s.d_model + s.d_in_proj + s.conv_dim + s.d_inner)
    assert size(1, 32768) - size(1, 16384) >= 16384 * per_row
