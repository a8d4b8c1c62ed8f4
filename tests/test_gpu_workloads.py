"""The measured workloads at their stated sizes, against the CPU oracle.

* Batch-1 decode of the 48-layer model as the benchmark times it: a 16-token
  prompt, then 256 greedy tokens in ONE launch of the persistent kernel's
  plain instantiation.  A second engine replays the same tokens one traced
  launch at a time; its argmax must pick the first engine's token at every
  step and its final state must equal the first engine's bit for bit, and
  the oracle follows the traced run (int8 codes taken where they are correct
  roundings) at 1e-3, with the exported int32 scaffold sums checked exactly.
* Prefill of one 2048-token sequence through all 48 layers: the oracle
  decodes the 2048 tokens one by one and the final conv/SSM states and the
  last logits must agree at 1e-3; the traced prefill equals, bit for bit,
  sequence 0 of the 8 x 2048 prefill in the benchmark's launch configuration.
* One 1.3B-shaped layer over 2 x 2048 token rows (the many-row LoRA-down
  kernel), sums exact and outputs at 1e-3.
* Batch-32 decode: 128 greedy steps replayed from the cached hipGraph as the
  benchmark times them; a traced eager follower reproduces every token and
  the final states bit for bit, and the oracle follows three sequences.

Long loops print progress (visible with -s) so a slow oracle is not taken
for a hang."""
import sys
import time

import numpy as np
import pytest

import oracle
import synth
from tests._common import (LONG_RUN_TIE_BAND, assert_close, assert_flip_fraction, check_acc, engine,
                           explain_rejection, follow_prefill, new_flip_stats, oracle_follow_step, token_ok,
                           trace_to_numpy)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


_MODELS = {}


def _full(seed):
    """(shape, oracle model) of the 48-layer model drawn with `seed` (cached per module)."""
    if seed not in _MODELS:
        s = synth.FULL_1P3B
        _MODELS.clear()  # hold one 48-layer oracle model at a time
        _MODELS[seed] = (s, oracle.Model(s, synth.gen_model(s, seed)))
    return _MODELS[seed]


def _states_equal(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# batch 1, 16 + 256 tokens, the timed kernel
# ---------------------------------------------------------------------------

@pytest.mark.timeout(1800)
def test_batch1_timed_launch_matches_traced_replay_and_oracle():
    seed = synth.SEED_BASE + 2  # the batch-1 benchmark's model and prompt
    s, om = _full(seed)
    prompt = synth.gen_tokens(seed, 0, 16, s.vocab)
    n = 256
    # engine A: what the benchmark times -- prefill, then all n tokens in one plain launch
    a = engine(s)
    a.set_path("persistent")
    a.load_synthetic(seed)
    lg_a, nx_a = a.prefill(_i32(prompt[None]))
    first = int(nx_a.cpu().numpy()[0])
    st_a_prefill = a.get_state(0)
    tok = _i32([first])
    out = a.generate(tok, n).cpu().numpy()[:, 0]
    st_a = a.get_state(0)
    a.check()
    a.close()
    _say(f"plain launch: {n} tokens")
    # engine B: the same prefill traced, then the same tokens one traced launch at a time
    b = engine(s)
    b.set_path("persistent")
    b.load_synthetic(seed)
    trp = trace_to_numpy(b.trace_prefill(_i32(prompt[None])))
    assert np.array_equal(trp["logits"][0], lg_a.cpu().numpy()[0])
    assert _states_equal(b.get_state(0), st_a_prefill)
    stats = new_flip_stats()
    st, ol = follow_prefill(om, s, prompt[None], trp, 0, 16, check_h_at={0, 15}, what="prompt", stats=stats)
    assert_close(trp["logits"][0], ol, what="prompt last logits")
    assert token_ok(first, ol)
    cur = first
    for i in range(n):
        tr = trace_to_numpy(b.trace_step(_i32([cur])))
        assert int(np.argmax(tr["logits"][0])) == int(out[i]), f"step {i}: traced argmax differs from the plain launch"
        hs, ol, otok = oracle_follow_step(om, st, cur, tr, stats=stats)
        assert_close(tr["logits"][0], ol, what=f"logits step {i}")
        assert token_ok(int(out[i]), ol), (i, int(out[i]), otok)
        if i in (0, 127, n - 1):
            for l in range(s.n_layer + 1):
                assert_close(tr["h"][l, 0], hs[l], what=f"h step {i} layer {l}")
            check_acc(om, tr, rows=[0], layers=range(s.n_layer), what=f"step {i}")
        if i % 64 == 63:
            _say(f"followed {i + 1} of {n} decode steps")
        cur = int(out[i])
    st_b = b.get_state(0)
    b.check()
    b.close()
    assert _states_equal(st_b, st_a), "traced replay's final state differs from the plain launch's"
    assert_close(st_a[1], st.ssm, what="ssm state after 16 + 256 tokens")
    assert_close(st_a[0], st.conv, what="conv state after 16 + 256 tokens")
    assert_flip_fraction(stats, "batch-1 16 + 256")
    _say(f"flips {stats['flips']} of {stats['codes']} codes")


# ---------------------------------------------------------------------------
# prefill 2048 tokens through 48 layers
# ---------------------------------------------------------------------------

@pytest.mark.timeout(2400)
def test_prefill_2048_tokens_48_layers_follows_oracle():
    seed = synth.SEED_BASE + 4  # the 8 x 2048 prefill benchmark's model and tokens
    s, om = _full(seed)
    B, T = 8, 2048
    toks = synth.gen_tokens(seed, 0, B * T, s.vocab).reshape(B, T)
    one = np.ascontiguousarray(toks[:1])
    eng = engine(s)
    eng.load_synthetic(seed)
    tr = trace_to_numpy(eng.trace_prefill(_i32(one)))
    st_g = eng.get_state(0)
    eng.check()
    eng.close()
    _say("traced prefill of 2048 tokens done; oracle follows")
    stats = new_flip_stats()
    st = oracle.State(s)
    h = None
    check_at = {0, 1, 63, 64, 1024, T - 1}
    for t in range(T):
        h = om.embed(int(one[0, t]))
        for l in range(s.n_layer):
            if t in check_at:
                assert_close(tr["h"][l, t], h, what=f"h token {t} layer {l}")
            keep = (st.conv[l].copy(), st.ssm[l].copy())
            try:
                h = oracle.layer_step(s, om.weights["layers"][l], h, st.conv[l], st.ssm[l],
                                      q1_force=tr["q1"][l, t], q2_force=tr["q2"][l, t], stats=stats,
                                      delta=LONG_RUN_TIE_BAND)
            except oracle.ForcedCodeError as e:
                raise AssertionError(f"token {t} layer {l}: {e}; "
                                     + explain_rejection(s, om.weights["layers"][l], h, keep, tr["q1"][l, t],
                                                         tr["q2"][l, t], tr["h"][l, t])) from e
        if t % 256 == 255:
            _say(f"oracle at token {t + 1} of {T}")
    _, ol, _, _ = om.lm_head(h, qf_force=tr["qf"][0], stats=stats, delta=LONG_RUN_TIE_BAND)
    assert_close(tr["logits"][0], ol, what="last logits")
    assert token_ok(int(np.argmax(tr["logits"][0])), ol)
    for l in range(s.n_layer):
        assert_close(st_g[1][l], st.ssm[l], what=f"ssm state layer {l}")
        assert_close(st_g[0][l], st.conv[l], what=f"conv state layer {l}")
    assert_flip_fraction(stats, "prefill 2048 x 48 layers")
    del tr
    # the benchmark's launch configuration: 8 sequences in one 16384-row chunk
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    eng.reset_state(B)
    lg, _ = eng.prefill(_i32(toks))
    assert _states_equal(eng.get_state(0), st_g), "sequence 0 of the 8 x 2048 prefill differs from its traced prefill"
    assert_close(lg.cpu().numpy()[0], ol, what="8 x 2048 prefill, sequence 0 last logits")
    eng.check()
    eng.close()


def test_layer_prefill_4096_rows_many_row_lora_down():
    # 2 x 2048 token rows on one 1.3B-shaped layer: M >= 4096 takes the
    # matrix-core LoRA-down kernel; exact scaffold sums, outputs and states at 1e-3
    s = synth.LAYER_1P3B
    seed = synth.SEED_BASE + 16
    B, T = 2, 2048
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    om = oracle.Model(s, synth.gen_model(s, seed))
    toks = synth.gen_tokens(seed, 17, B * T, s.vocab).reshape(B, T)
    tr = trace_to_numpy(eng.trace_prefill(_i32(toks), want_acc=True))
    stats = new_flip_stats()
    for b in range(B):
        st, ol = follow_prefill(om, s, toks, tr, b, T, check_h_at={0, 1, 64, 2047}, what="M=4096", stats=stats)
        assert_close(tr["logits"][b], ol, what=f"last logits seq {b}")
        conv_g, ssm_g = eng.get_state(b)
        assert_close(ssm_g, st.ssm, what=f"ssm state seq {b}")
        assert_close(conv_g, st.conv, what=f"conv state seq {b}")
    check_acc(om, tr, rows=[0, 1, 2047, 2048, 3000, 4095], layers=[0], what="M=4096")
    assert_flip_fraction(stats, "M=4096")
    eng.check()
    eng.close()


# ---------------------------------------------------------------------------
# batch 32, 8-token prompts, 128 steps of graph replay
# ---------------------------------------------------------------------------

@pytest.mark.timeout(1800)
def test_batch32_graph_replay_128_steps():
    seed = synth.SEED_BASE + 3  # the batch-32 benchmark's model and prompts
    s, om = _full(seed)
    B, T, n = 32, 8, 128
    follow = (0, 13, 31)
    toks = synth.gen_tokens(seed, 0, B * T, s.vocab).reshape(B, T)
    # engine A: prefill, then n steps replayed from the cached graph (as timed)
    a = engine(s, max_batch=B)
    a.load_synthetic(seed)
    lg_a, nx_a = a.prefill(_i32(toks))
    start = nx_a.clone()
    out = a.generate(nx_a, n, use_graph=True).cpu().numpy()
    st_a = [a.get_state(q) for q in range(B)]
    a.check()
    a.close()
    _say(f"graph replay: {n} steps at batch {B}")
    # engine B: traced prefill and eager traced steps on the same tokens
    b = engine(s, max_batch=B)
    b.load_synthetic(seed)
    trp = trace_to_numpy(b.trace_prefill(_i32(toks)))
    assert np.array_equal(trp["logits"], lg_a.cpu().numpy())
    stats = new_flip_stats()
    sts = {}
    for q in follow:
        sts[q], ol = follow_prefill(om, s, toks, trp, q, T, what="prompt", stats=stats)
        assert_close(trp["logits"][q], ol, what=f"prompt logits seq {q}")
    cur = start.cpu().numpy().tolist()
    for i in range(n):
        tr = trace_to_numpy(b.trace_step(_i32(cur), want_acc=(i in (0, n - 1))))
        assert np.array_equal(np.argmax(tr["logits"], axis=1), out[i]), f"step {i}: eager argmax differs from replay"
        for q in follow:
            _, ol, otok = oracle_follow_step(om, sts[q], cur[q], tr, q, stats=stats)
            assert_close(tr["logits"][q], ol, what=f"logits step {i} seq {q}")
            assert token_ok(int(out[i, q]), ol), (i, q, int(out[i, q]), otok)
        if i in (0, n - 1):
            check_acc(om, tr, rows=list(follow), layers=(0, 24, 47), what=f"step {i}")
        if i % 32 == 31:
            _say(f"followed {i + 1} of {n} steps")
        cur = out[i].tolist()
    for q in range(B):
        assert _states_equal(b.get_state(q), st_a[q]), f"seq {q}: eager follower state differs from graph replay"
    for q in follow:
        assert_close(st_a[q][1], sts[q].ssm, what=f"ssm state seq {q}")
        assert_close(st_a[q][0], sts[q].conv, what=f"conv state seq {q}")
    assert_flip_fraction(stats, "batch 32, 128 steps")
    b.check()
    b.close()
