"""Special cases of the method on the device, on every path that serves them
(batch-1 persistent kernel, per-layer GEMV kernels, the batched path's decode
step, and prefill with the sequential or the chunked matrix-core scan):

* dt = 0 (dt_bias = -1e4, softplus underflows to 0, exp(0) = 1): the SSM
  state is left bit for bit as it was;
* a decay that underflows (A_log = 60, exp(-dt e^60) = 0): the step is
  memoryless, so two different prior SSM states give bit-identical results;
* an exact tie of two logits (two identical embedding rows and scales): the
  lower vocabulary index wins, whichever side of the maximum it sits;
* an all-zero gate (the z rows of in_proj scaled by 0): the gated output is
  zero, its int8 codes and scale are zero, and the layer adds exactly nothing
  to the residual stream.

Each case is also followed by the oracle where it produces floating outputs."""
import numpy as np
import pytest

import oracle
import synth
from tests._common import assert_close, engine, follow_prefill, oracle_follow_step, trace_to_numpy

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# a 2-layer stack at the 1.3B layer shape (the persistent kernel needs >= 2 layers)
TWO_1P3B = synth.Shape(n_layer=2, d_model=2048, d_inner=4096, d_state=128, headdim=64, vocab=1024)
SHAPES = [synth.TINY, TWO_1P3B]
MODES = ["persistent", "kernels", "gemm", "prefill"]
T_PREFILL = 70  # a whole 64-token chunk of the chunked scan and a padded ragged one


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _setup(shape, mode, seed):
    eng = engine(shape)
    eng.set_path("auto" if mode == "prefill" else mode)
    eng.load_synthetic(seed)
    return eng


def _run(eng, mode, toks):
    """One step (or the prefill) from the engine's current state; returns (logits, next token)."""
    if mode == "prefill":
        lg, nx = eng.prefill(_i32(toks[None]))
    else:
        lg, nx = eng.decode_step(_i32(toks[:1]))
    return lg.cpu().numpy()[0], int(nx.cpu().numpy()[0])


def _trace(eng, mode, toks):
    if mode == "prefill":
        return trace_to_numpy(eng.trace_prefill(_i32(toks[None])))
    return trace_to_numpy(eng.trace_step(_i32(toks[:1])))


def _random_state(shape, seed):
    rng = np.random.default_rng(seed)
    conv = rng.standard_normal((shape.n_layer, shape.conv_dim, shape.d_conv - 1)).astype(np.float32)
    ssm = (rng.standard_normal((shape.n_layer, shape.n_heads, shape.headdim, shape.d_state)) * 0.5).astype(np.float32)
    return conv, ssm


def _weights_with(shape, seed, changes):
    w = synth.gen_model(shape, seed)
    for (l, k), v in changes.items():
        w["layers"][l][k] = v
    return w


def _follow(shape, w, mode, toks, tr, conv, ssm):
    """Oracle run from the given state on the GPU's int8 codes; returns (oracle state, last logits)."""
    om = oracle.Model(shape, w)
    st = oracle.State(shape)
    st.conv[:] = conv
    st.ssm[:] = ssm
    if mode == "prefill":
        return follow_prefill(om, shape, toks[None], tr, 0, toks.size, st=st)
    _, ol, _ = oracle_follow_step(om, st, int(toks[0]), tr)
    return st, ol


@pytest.mark.parametrize("shape", SHAPES, ids=["tiny", "1p3b"])
@pytest.mark.parametrize("mode", MODES)
def test_dt_zero_leaves_state_bit_identical(shape, mode):
    seed = synth.SEED_BASE + 40
    eng = _setup(shape, mode, seed)
    dtb = np.full(shape.n_heads, -1e4, np.float32)
    for l in range(shape.n_layer):
        eng.set_tensor(l, "dt_bias", dtb)
    conv, ssm = _random_state(shape, 1)
    toks = synth.gen_tokens(seed, 1, T_PREFILL if mode == "prefill" else 1, shape.vocab)
    eng.set_state(0, conv, ssm)
    _run(eng, mode, toks)  # the plain kernels
    assert np.array_equal(eng.get_state(0)[1], ssm), "SSM state moved with dt = 0"
    eng.set_state(0, conv, ssm)
    tr = _trace(eng, mode, toks)  # the tracing kernels, followed by the oracle
    conv_g, ssm_g = eng.get_state(0)
    assert np.array_equal(ssm_g, ssm)
    w = _weights_with(shape, seed, {(l, "dt_bias"): dtb for l in range(shape.n_layer)})
    st, ol = _follow(shape, w, mode, toks, tr, conv, ssm)
    assert np.array_equal(st.ssm, ssm.astype(np.float64))  # the oracle's own dt = 0 case
    assert_close(tr["logits"][0], ol, what="logits")
    assert_close(conv_g, st.conv, what="conv state")
    eng.check()
    eng.close()


@pytest.mark.parametrize("shape", SHAPES, ids=["tiny", "1p3b"])
@pytest.mark.parametrize("mode", MODES + ["prefill6", "prefill130"])
def test_underflowing_decay_is_memoryless(shape, mode):
    # prefill6 / prefill130: one padded chunk, two whole chunks and a padded one
    seed = synth.SEED_BASE + 41
    T = {"prefill6": 6, "prefill130": 130}.get(mode, T_PREFILL)
    mode = "prefill" if mode.startswith("prefill") else mode
    eng = _setup(shape, mode, seed)
    alog = np.full(shape.n_heads, 60.0, np.float32)
    for l in range(shape.n_layer):
        eng.set_tensor(l, "A_log", alog)
    conv, ssm1 = _random_state(shape, 2)
    _, ssm2 = _random_state(shape, 3)
    toks = synth.gen_tokens(seed, 2, T if mode == "prefill" else 1, shape.vocab)
    res = []
    for ssm in (ssm1, ssm2):
        eng.set_state(0, conv, ssm)
        lg, nx = _run(eng, mode, toks)
        res.append((lg, nx, eng.get_state(0)))
    assert np.array_equal(res[0][0], res[1][0]) and res[0][1] == res[1][1], "logits depend on the prior SSM state"
    sa, sb = res[0][2][1], res[1][2][1]
    assert np.isfinite(sa).all() and np.isfinite(sb).all(), f"non-finite SSM state: {int((~np.isfinite(sa)).sum())}"
    if not np.array_equal(sa, sb):
        diff = ~((sa == sb) | (np.isnan(sa) & np.isnan(sb)))
        per_layer = [int(diff[l].sum()) for l in range(shape.n_layer)]
        idx = np.argwhere(diff)[:4].tolist()
        raise AssertionError(f"SSM state depends on the prior SSM state: differing elements per layer {per_layer}, "
                             f"NaN {int(np.isnan(sa).sum())}/{int(np.isnan(sb).sum())}, first {idx}, "
                             f"values {[(float(sa[tuple(i)]), float(sb[tuple(i)])) for i in idx]}")
    eng.set_state(0, conv, ssm1)
    tr = _trace(eng, mode, toks)
    w = _weights_with(shape, seed, {(l, "A_log"): alog for l in range(shape.n_layer)})
    st, ol = _follow(shape, w, mode, toks, tr, conv, ssm1)
    assert_close(tr["logits"][0], ol, what="logits")
    assert_close(eng.get_state(0)[1], st.ssm, what="ssm state")
    eng.check()
    eng.close()


@pytest.mark.parametrize("shape", SHAPES, ids=["tiny", "1p3b"])
@pytest.mark.parametrize("mode", MODES)
def test_exact_logit_tie_takes_lowest_index(shape, mode):
    seed = synth.SEED_BASE + 42
    eng = _setup(shape, mode, seed)
    toks = synth.gen_tokens(seed, 3, T_PREFILL if mode == "prefill" else 1, shape.vocab)
    eng.reset_state(1)
    lg, nx = _run(eng, mode, toks)
    a = int(np.argmax(lg))
    assert nx == a
    E, sE = eng.get_tensor(-1, "E"), eng.get_tensor(-1, "sE")
    used = set(int(t) for t in toks)
    lower = [v for v in range(a) if v not in used]
    higher = [v for v in range(a + 1, shape.vocab) if v not in used]
    for other, winner in ([(lower[0], lower[0])] if lower else []) + [(higher[-1], a)]:
        E2, sE2 = E.copy(), sE.copy()
        E2[other], sE2[other] = E[a], sE[a]
        eng.set_tensor(-1, "E", E2)
        eng.set_tensor(-1, "sE", sE2)
        eng.reset_state(1)
        lg2, nx2 = _run(eng, mode, toks)
        assert lg2[other] == lg2[a] == lg[a], "duplicated rows must give the same logit bit for bit"
        assert nx2 == winner, (other, a, nx2)
    eng.check()
    eng.close()


@pytest.mark.parametrize("shape", SHAPES, ids=["tiny", "1p3b"])
@pytest.mark.parametrize("mode", MODES)
def test_zero_gate_adds_nothing(shape, mode):
    seed = synth.SEED_BASE + 43
    eng = _setup(shape, mode, seed)
    sw = eng.get_tensor(0, "in_sw").copy()
    sb = eng.get_tensor(0, "in_sB").copy()
    sw[:shape.d_inner] = 0.0  # rows z: zero scaffold and LoRA scales, so z = 0 exactly
    sb[:shape.d_inner] = 0.0
    eng.set_tensor(0, "in_sw", sw)
    eng.set_tensor(0, "in_sB", sb)
    toks = synth.gen_tokens(seed, 4, T_PREFILL if mode == "prefill" else 1, shape.vocab)
    conv, ssm = _random_state(shape, 4)
    eng.set_state(0, conv, ssm)
    tr = _trace(eng, mode, toks)
    assert not tr["q2"][0].any(), "the gated output of layer 0 must quantise to zero codes"
    h0, h1 = tr["h"][0], tr["h"][1]
    if mode == "persistent":
        # the residual hop carries a 2-bit write count in the lowest mantissa
        # bit of each value: equal up to that bit
        m = np.uint32(0xFFFFFFFE)
        assert np.array_equal(h0.view(np.uint32) & m, h1.view(np.uint32) & m)
    else:
        assert np.array_equal(h0, h1), "layer 0 must leave the residual stream unchanged"
    w = _weights_with(shape, seed, {(0, "in_sw"): sw, (0, "in_sB"): sb})
    st, ol = _follow(shape, w, mode, toks, tr, conv, ssm)
    assert_close(tr["logits"][0], ol, what="logits")
    eng.check()
    eng.close()


@pytest.mark.parametrize("shape", SHAPES, ids=["tiny", "1p3b"])
def test_persistent_result_independent_of_launch_history(shape):
    # the same step from the same state gives the same bits however many
    # tokens were decoded in between (the mailboxes' write count differs)
    seed = synth.SEED_BASE + 44
    eng = _setup(shape, "persistent", seed)
    conv, ssm = _random_state(shape, 5)
    toks = synth.gen_tokens(seed, 5, 1, shape.vocab)
    outs = []
    for extra in (0, 1, 2, 3, 5):
        if extra:
            eng.generate(_i32(toks), extra)
        eng.set_state(0, conv, ssm)
        lg, nx = _run(eng, "persistent", toks)
        outs.append((lg, nx, eng.get_state(0)))
    for lg, nx, st in outs[1:]:
        assert np.array_equal(lg, outs[0][0]) and nx == outs[0][1]
        assert np.array_equal(st[0], outs[0][2][0]) and np.array_equal(st[1], outs[0][2][1])
    eng.check()
    eng.close()
