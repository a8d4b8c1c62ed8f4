"""Parity of the batched path (int8 matrix-core GEMMs, causal conv over T,
the scan token by token or in 64-token chunks on the fp32 matrix cores)
against the CPU oracle: the GEMM kernel bit-exact on its integer sums,
batched decode and traced prefill teacher-forced on the GPU's int8 codes, at
the tiny shape, one 1.3B-shaped layer (2048 tokens; ragged chunks continued
from a state) and the 48-layer model."""
import numpy as np
import pytest

import oracle
import synth
from tests._common import assert_close, engine, follow_prefill, oracle_follow_step, token_ok, trace_to_numpy

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


# ---------------------------------------------------------------------------
# the GEMM kernel
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,d_in,d_out", [(1, 256, 1072), (3, 512, 256), (32, 2048, 8512), (33, 2048, 333),
                                          (130, 4096, 2048), (257, 256, 64), (5, 8192, 64), (300, 128, 7)])
def test_k_gemm_matches_oracle(M, d_in, d_out):
    from bit_quantized_mamba_amd import k_gemm
    rng = np.random.default_rng(M * 131 + d_in * 7 + d_out)
    r = 16
    bits = rng.integers(0, 2**32, size=(d_out, d_in // 32), dtype=np.uint64).astype(np.uint32)
    sw = rng.uniform(0.01, 0.05, d_out).astype(np.float32)
    A = rng.integers(-127, 128, size=(r, d_in)).astype(np.int8)
    sA = rng.uniform(5e-4, 2e-3, r).astype(np.float32)
    Bm = rng.integers(-127, 128, size=(d_out, r)).astype(np.int8)
    sB = rng.uniform(5e-4, 2e-3, d_out).astype(np.float32)
    q = rng.integers(-127, 128, size=(M, d_in)).astype(np.int8)
    q[0, :5] = 127
    q[-1, -3:] = -127
    s = rng.uniform(0.01, 0.05, M).astype(np.float32)
    acc, y = k_gemm(_dev(bits), _dev(sw), _dev(A), _dev(sA), _dev(Bm), _dev(sB), _dev(q), _dev(s))
    acc, y = acc.cpu().numpy(), y.cpu().numpy()
    # integer sums: numpy int64 matmul of the unpacked +-1 matrix, all rows
    W = np.where(np.unpackbits(bits.view(np.uint8), bitorder="little").reshape(d_out, d_in), 1, -1)
    want = q.astype(np.int64) @ W.T.astype(np.int64)
    assert np.array_equal(acc, want)
    for m in sorted({0, M // 2, M - 1}):
        yo, acco, _ = oracle.proj(bits, sw, A, sA, Bm, sB, q[m], s[m])
        assert np.array_equal(acc[m], acco), m
        assert_close(y[m], yo, what=f"y[{m}]")


def test_k_gemm_sign_probes():
    from bit_quantized_mamba_amd import k_gemm
    d_in, d_out, r = 2048, 96, 16
    rng = np.random.default_rng(5)
    z = np.zeros
    ones = lambda n: np.ones(n, np.float32)  # noqa: E731
    bits = np.zeros((d_out, d_in // 32), dtype=np.uint32)
    bits[: d_out // 2] = 0xFFFFFFFF
    q = rng.integers(-127, 128, size=(40, d_in)).astype(np.int8)
    acc, _ = k_gemm(_dev(bits), _dev(ones(d_out)), _dev(z((r, d_in), np.int8)), _dev(ones(r)),
                    _dev(z((d_out, r), np.int8)), _dev(ones(d_out)), _dev(q), _dev(ones(40)))
    acc = acc.cpu().numpy()
    tot = q.astype(np.int64).sum(axis=1)
    assert np.all(acc[:, : d_out // 2] == tot[:, None]) and np.all(acc[:, d_out // 2:] == -tot[:, None])
    bits = rng.integers(0, 2**32, size=(d_out, d_in // 32), dtype=np.uint64).astype(np.uint32)
    cols = [0, 31, 32, 63, 64, 1000, 2047]
    q = np.zeros((len(cols), d_in), dtype=np.int8)
    for i, j in enumerate(cols):
        q[i, j] = 127
    acc, _ = k_gemm(_dev(bits), _dev(ones(d_out)), _dev(z((r, d_in), np.int8)), _dev(ones(r)),
                    _dev(z((d_out, r), np.int8)), _dev(ones(d_out)), _dev(q), _dev(ones(len(cols))))
    acc = acc.cpu().numpy()
    for i, j in enumerate(cols):
        want = np.where((bits[:, j // 32] >> np.uint32(j % 32)) & 1, 127, -127)
        assert np.array_equal(acc[i], want), j


# ---------------------------------------------------------------------------
# decode on the batched path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B,steps", [(1, 24), (4, 12)])
def test_tiny_decode_on_gemm_path(B, steps):
    s = synth.TINY
    seed = synth.SEED_BASE
    eng = engine(s, max_batch=B)
    eng.set_path("gemm")
    eng.load_synthetic(seed)
    om = oracle.Model(s, synth.gen_model(s, seed))
    sts = [oracle.State(s) for _ in range(B)]
    toks = [int(t) for t in synth.gen_tokens(seed, 6, B, s.vocab)]
    for step in range(steps):
        tr = trace_to_numpy(eng.trace_step(_i32(toks)))
        for b in range(B):
            hs, ol, otok = oracle_follow_step(om, sts[b], toks[b], tr, b)
            for l in range(s.n_layer + 1):
                assert_close(tr["h"][l, b], hs[l], what=f"h step {step} seq {b} layer {l}")
            assert_close(tr["logits"][b], ol, what=f"logits step {step} seq {b}")
            gtok = int(np.argmax(tr["logits"][b]))
            assert token_ok(gtok, ol), (step, b, gtok, otok)
            toks[b] = gtok
    for b in range(B):
        conv_g, ssm_g = eng.get_state(b)
        assert_close(conv_g, sts[b].conv, what=f"conv state seq {b}")
        assert_close(ssm_g, sts[b].ssm, what=f"ssm state seq {b}")
    eng.check()
    eng.close()


@pytest.mark.parametrize("B", [1, 3])
def test_1p3b_layer_decode_on_gemm_path(B):
    # one 1.3B-shaped layer: the decode-sized GEMM (K 2048 / 4096, conv in its
    # epilogue) and the single-token scan at headdim 64, d_state 128
    s = synth.LAYER_1P3B
    seed = synth.SEED_BASE + 5
    eng = engine(s, max_batch=B)
    eng.set_path("gemm")
    eng.load_synthetic(seed)
    om = oracle.Model(s, synth.gen_model(s, seed))
    sts = [oracle.State(s) for _ in range(B)]
    toks = [int(t) for t in synth.gen_tokens(seed, 11, B, s.vocab)]
    for step in range(6):
        tr = trace_to_numpy(eng.trace_step(_i32(toks)))
        for b in range(B):
            hs, ol, otok = oracle_follow_step(om, sts[b], toks[b], tr, b)
            assert_close(tr["h"][1, b], hs[1], what=f"h step {step} seq {b}")
            assert_close(tr["logits"][b], ol, what=f"logits step {step} seq {b}")
            toks[b] = int(np.argmax(tr["logits"][b]))
    for b in range(B):
        conv_g, ssm_g = eng.get_state(b)
        assert_close(conv_g, sts[b].conv, what=f"conv state seq {b}")
        assert_close(ssm_g, sts[b].ssm, what=f"ssm state seq {b}")
    eng.check()
    eng.close()


def test_decode_across_gemm_kernels_matches_single_sequences():
    # 65 sequences split into chains of 33 (tiled matrix-core GEMMs, a ragged
    # 128-row tile) and 32 (the skinny GEMM); a sequence decoded alone runs
    # the skinny GEMM at M = 1.  Integer sums are exact either way; the float
    # epilogues must agree with the one-sequence run to the 1e-3 metric
    # whichever kernel served the sequence, and bit for bit within a kernel.
    s = synth.Shape(n_layer=2, d_model=2048, d_inner=4096, d_state=128, headdim=64, vocab=1024)
    seed = synth.SEED_BASE + 41
    B = 65
    toks = synth.gen_tokens(seed, 12, B, s.vocab).astype(np.int32)
    big = engine(s, max_batch=B)
    big.set_path("gemm")
    big.load_synthetic(seed)
    one = engine(s, max_batch=1)
    one.set_path("gemm")
    one.load_synthetic(seed)
    lg_b, ins = [], []
    t = toks.copy()
    for step in range(3):
        ins.append(t.copy())
        lg, nx = big.decode_step(_i32(t))
        lg_b.append(lg.cpu().numpy())
        t = nx.cpu().numpy().astype(np.int32)
    for b in (0, 32, 33, 64):
        one.reset_state(1)
        for step in range(3):  # the batch run's inputs (greedy tokens could part near a tie)
            lg, _ = one.decode_step(_i32(ins[step][b:b + 1]))
            lg1 = lg.cpu().numpy()[0]
            assert_close(lg1, lg_b[step][b], what=f"logits seq {b} step {step}")
            if b >= 33:  # the skinny-GEMM chain: the same kernels as the single run
                assert np.array_equal(lg1.view(np.uint32), lg_b[step][b].view(np.uint32)), (b, step)
        conv1, ssm1 = one.get_state(0)
        convb, ssmb = big.get_state(b)
        assert_close(ssm1, ssmb, what=f"ssm state seq {b}")
        assert_close(conv1, convb, what=f"conv state seq {b}")
    big.check()
    big.close()
    one.close()


# ---------------------------------------------------------------------------
# traced prefill
# ---------------------------------------------------------------------------

def _follow_prefill(om, s, toks, tr, b, T, check_h_at=(), h_tol_what="", st=None):
    return follow_prefill(om, s, toks, tr, b, T, check_h_at=check_h_at, what=h_tol_what, st=st)


@pytest.mark.parametrize("B,T", [(3, 37), (1, 1), (2, 64)])
def test_tiny_traced_prefill(B, T):
    s = synth.TINY
    seed = synth.SEED_BASE + 3
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    om = oracle.Model(s, synth.gen_model(s, seed))
    toks = synth.gen_tokens(seed, 7, B * T, s.vocab).reshape(B, T)
    tr = trace_to_numpy(eng.trace_prefill(_i32(toks)))
    for b in range(B):
        st, ol = _follow_prefill(om, s, toks, tr, b, T, check_h_at=set(range(T)))
        assert_close(tr["logits"][b], ol, what=f"last logits seq {b}")
        conv_g, ssm_g = eng.get_state(b)
        assert_close(conv_g, st.conv, what=f"conv state seq {b}")
        assert_close(ssm_g, st.ssm, what=f"ssm state seq {b}")
    eng.check()
    eng.close()


def test_one_1p3b_layer_prefill_2048_tokens():
    # the prefill sequence length of the 8 x 2048 workload, on one 1.3B-shaped layer
    s = synth.LAYER_1P3B
    seed = synth.SEED_BASE + 4
    B, T = 1, 2048
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    om = oracle.Model(s, synth.gen_model(s, seed))
    toks = synth.gen_tokens(seed, 8, B * T, s.vocab).reshape(B, T)
    tr = trace_to_numpy(eng.trace_prefill(_i32(toks)))
    for b in range(B):
        st = oracle.State(s)
        hout = np.empty((T, s.d_model))
        for t in range(T):
            m = b * T + t
            h = om.embed(int(toks[b, t]))
            hout[t] = oracle.layer_step(s, om.weights["layers"][0], h, st.conv[0], st.ssm[0],
                                        q1_force=tr["q1"][0, m], q2_force=tr["q2"][0, m])
        got = tr["h"][1, b * T:(b + 1) * T]
        for t in (0, 1, 2, 3, 100, 1023, 2047):
            assert_close(got[t], hout[t], what=f"seq {b} token {t}")
        assert_close(got, hout, what=f"seq {b} all tokens")
        conv_g, ssm_g = eng.get_state(b)
        assert_close(conv_g, st.conv, what=f"conv state seq {b}")
        assert_close(ssm_g, st.ssm, what=f"ssm state seq {b}")
    eng.close()


def test_1p3b_layer_prefill_ragged_chunks_continue_from_state():
    # Two sequences on one 1.3B-shaped layer: a prefill of 70 tokens (a whole
    # 64-token chunk of the chunked scan and a ragged one), then 100 more
    # tokens from the state it left (a nonzero initial state, a ragged last
    # chunk).  Outputs and states follow the oracle token by token.
    s = synth.LAYER_1P3B
    seed = synth.SEED_BASE + 11
    B, T1, T2 = 2, 70, 100
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    om = oracle.Model(s, synth.gen_model(s, seed))
    toks = synth.gen_tokens(seed, 12, B * (T1 + T2), s.vocab).reshape(B, T1 + T2)
    first, second = np.ascontiguousarray(toks[:, :T1]), np.ascontiguousarray(toks[:, T1:])
    tr1 = trace_to_numpy(eng.trace_prefill(_i32(first)))
    mid = [eng.get_state(b) for b in range(B)]
    tr2 = trace_to_numpy(eng.trace_prefill(_i32(second)))
    for b in range(B):
        st, _ = _follow_prefill(om, s, first, tr1, b, T1, check_h_at={0, 1, 63, 64, 69})
        assert_close(mid[b][1], st.ssm, what=f"ssm state seq {b} after {T1} tokens")
        assert_close(mid[b][0], st.conv, what=f"conv state seq {b} after {T1} tokens")
        st, ol = _follow_prefill(om, s, second, tr2, b, T2, check_h_at={0, 1, 63, 64, 99}, st=st)
        assert_close(tr2["logits"][b], ol, what=f"last logits seq {b}")
        conv_g, ssm_g = eng.get_state(b)
        assert_close(ssm_g, st.ssm, what=f"ssm state seq {b} after {T1 + T2} tokens")
        assert_close(conv_g, st.conv, what=f"conv state seq {b} after {T1 + T2} tokens")
    eng.check()
    eng.close()


@pytest.mark.parametrize("B,T1,T2", [(1, 2, 64), (3, 65, 129), (2, 64, 1)])
def test_1p3b_layer_prefill_chunk_edges(B, T1, T2):
    # Lengths at the edges of the 64-token chunks of the matrix-core scan (2,
    # 64, 65, 129 tokens), several sequences per launch, and a second prefill
    # from the state the first one left (T2 = 1 takes the decode-step scan).
    s = synth.LAYER_1P3B
    seed = synth.SEED_BASE + 13
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    om = oracle.Model(s, synth.gen_model(s, seed))
    toks = synth.gen_tokens(seed, 14 + T1, B * (T1 + T2), s.vocab).reshape(B, T1 + T2)
    first, second = np.ascontiguousarray(toks[:, :T1]), np.ascontiguousarray(toks[:, T1:])
    tr1 = trace_to_numpy(eng.trace_prefill(_i32(first)))
    tr2 = trace_to_numpy(eng.trace_prefill(_i32(second)))
    for b in range(B):
        st, _ = _follow_prefill(om, s, first, tr1, b, T1, check_h_at={0, T1 - 1})
        st, ol = _follow_prefill(om, s, second, tr2, b, T2, check_h_at={0, T2 - 1}, st=st)
        assert_close(tr2["logits"][b], ol, what=f"last logits seq {b}")
        conv_g, ssm_g = eng.get_state(b)
        assert_close(ssm_g, st.ssm, what=f"ssm state seq {b}")
        assert_close(conv_g, st.conv, what=f"conv state seq {b}")
    eng.check()
    eng.close()


@pytest.fixture(scope="module")
def full_model():
    s = synth.FULL_1P3B
    seed = synth.SEED_BASE + 2
    w = synth.gen_model(s, seed)
    return s, seed, w, oracle.Model(s, w)


def test_full_model_traced_prefill(full_model):
    s, seed, w, om = full_model
    B, T = 2, 12
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    toks = synth.gen_tokens(seed, 9, B * T, s.vocab).reshape(B, T)
    tr = trace_to_numpy(eng.trace_prefill(_i32(toks)))
    for b in range(B):
        st, ol = _follow_prefill(om, s, toks, tr, b, T, check_h_at={0, T - 1})
        assert_close(tr["logits"][b], ol, what=f"last logits seq {b}")
        gtok = int(np.argmax(tr["logits"][b]))
        assert token_ok(gtok, ol), (b, gtok, int(np.argmax(ol)))
        conv_g, ssm_g = eng.get_state(b)
        assert_close(ssm_g, st.ssm, what=f"ssm state seq {b}")
        assert_close(conv_g, st.conv, what=f"conv state seq {b}")
    eng.close()


def test_full_model_prefill_8x2048_batch_independence(full_model):
    # The 8 x 2048 prefill as the bench runs it (48 layers, one 16384-row
    # chunk): each sequence's last logits and final state equal, bit for bit,
    # those of a prefill of that sequence alone (every kernel treats rows and
    # sequences independently; the arithmetic is checked against the oracle
    # by the shorter prefills above).
    s, seed, w, om = full_model
    B, T = 8, 2048
    toks = synth.gen_tokens(seed, 15, B * T, s.vocab).reshape(B, T)
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    eng.reset_state(B)
    lg_b, nx_b = eng.prefill(_i32(toks))
    lg_b = lg_b.cpu().numpy()
    st_b = {b: eng.get_state(b) for b in (0, 5, 7)}
    eng.close()
    one = engine(s, max_batch=1)
    one.load_synthetic(seed)
    for b in (0, 5, 7):
        one.reset_state(1)
        lg_1, _ = one.prefill(_i32(toks[b:b + 1]))
        assert np.array_equal(lg_1.cpu().numpy()[0], lg_b[b]), b
        conv_1, ssm_1 = one.get_state(0)
        assert np.array_equal(ssm_1, st_b[b][1]) and np.array_equal(conv_1, st_b[b][0]), b
        assert np.all(np.isfinite(lg_b[b]))
    one.close()


@pytest.mark.parametrize("B,T,follow", [(32, 8, (0, 13, 31)), (512, 2, (0, 257, 511))])
def test_full_model_batched_decode_sampled(full_model, B, T, follow):
    # the batch-32 decode workload (32 sequences prefilled with 8 tokens) and
    # batch 512 (the skinny kernels give way to the tiled GEMMs, the LM head
    # runs in 16 launches of 32 sequences), then greedy steps; three sequences
    # are followed by the oracle
    s, seed, w, om = full_model
    eng = engine(s, max_batch=B)
    eng.load_synthetic(seed)
    toks = synth.gen_tokens(seed, 10, B * T, s.vocab).reshape(B, T)
    tr = trace_to_numpy(eng.trace_prefill(_i32(toks)))
    sts, nxt = {}, {}
    for b in follow:
        sts[b], ol = _follow_prefill(om, s, toks, tr, b, T)
        assert_close(tr["logits"][b], ol, what=f"prefill logits seq {b}")
    cur = [int(np.argmax(tr["logits"][b])) for b in range(B)]
    for step in range(3):
        trd = trace_to_numpy(eng.trace_step(_i32(cur)))
        for b in follow:
            hs, ol, otok = oracle_follow_step(om, sts[b], cur[b], trd, b)
            assert_close(trd["logits"][b], ol, what=f"decode step {step} seq {b}")
            assert token_ok(int(np.argmax(trd["logits"][b])), ol), (step, b)
        cur = [int(np.argmax(trd["logits"][b])) for b in range(B)]
    for b in follow:
        conv_g, ssm_g = eng.get_state(b)
        assert_close(ssm_g, sts[b].ssm, what=f"ssm state seq {b}")
    eng.check()
    eng.close()
