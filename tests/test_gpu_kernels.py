"""GPU kernel parity against the CPU oracle (bit-exact integers, 1e-3 floats)."""
import numpy as np
import pytest

import oracle
import synth
from tests._common import assert_close, engine

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


# ---------------------------------------------------------------------------
# device synthetic generator == host generator (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [synth.TINY, synth.LAYER_1P3B])
def test_device_generator_matches_host(shape):
    seed = synth.SEED_BASE + 1
    eng = engine(shape)
    eng.load_synthetic(seed)
    torch.cuda.synchronize()
    for l in range(shape.n_layer):
        for k in synth.LAYER_KINDS:
            want = synth.gen_layer_tensor(shape, seed, l, k)
            got = eng.get_tensor(l, k)
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (l, k)
    for k in synth.GLOBAL_KINDS:
        want = synth.gen_global_tensor(shape, seed, k)
        assert np.array_equal(eng.get_tensor(-1, k).view(np.uint8), want.view(np.uint8)), k
    eng.close()


def test_device_generator_full_model_samples():
    s = synth.FULL_1P3B
    seed = synth.SEED_BASE + 2
    eng = engine(s)
    eng.load_synthetic(seed)
    torch.cuda.synchronize()
    for l in (0, 47):
        for k in ("in_bits", "out_B", "conv_w", "D", "gnorm_w"):
            want = synth.gen_layer_tensor(s, seed, l, k)
            assert np.array_equal(eng.get_tensor(l, k).view(np.uint8), want.view(np.uint8)), (l, k)
    for k in ("sE", "final_norm"):
        assert np.array_equal(eng.get_tensor(-1, k), synth.gen_global_tensor(s, seed, k)), k
    E = eng.get_tensor(-1, "E")
    # a sample of embedding rows, drawn element by element
    rows = [0, 1, 25000, 50287]
    for r in rows:
        want = synth.gen_int8(seed, synth.GLOBAL_TID["E"], (r + 1) * s.d_model)[r * s.d_model:]
        assert np.array_equal(E[r], want), r
    eng.close()


# ---------------------------------------------------------------------------
# quantiser
# ---------------------------------------------------------------------------

def test_k_quant_bit_exact():
    from bit_quantized_mamba_amd import k_quant
    rng = np.random.default_rng(1)
    rows = [rng.standard_normal(2048).astype(np.float32) * 3,
            np.zeros(2048, dtype=np.float32),
            np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5] * 256, dtype=np.float32),
            (rng.standard_normal(2048) * 1e-30).astype(np.float32),
            rng.uniform(-1, 1, 2048).astype(np.float32)]
    u = np.stack(rows)
    q, s = k_quant(_dev(u))
    q, s = q.cpu().numpy(), s.cpu().numpy()
    for i, row in enumerate(rows):
        qo, so = oracle.quant_f32(row)
        assert np.array_equal(q[i], qo), i
        assert s[i] == so, i


# ---------------------------------------------------------------------------
# scaffold + LoRA projection
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_in,d_out,B", [(256, 1072, 1), (512, 256, 3), (2048, 8512, 1), (4096, 2048, 2),
                                          (2048, 333, 5), (8192, 64, 1), (128, 7, 2)])
def test_k_proj_matches_oracle(d_in, d_out, B):
    from bit_quantized_mamba_amd import k_proj
    rng = np.random.default_rng(d_in * 7 + d_out + B)
    r = 16
    bits = rng.integers(0, 2**32, size=(d_out, d_in // 32), dtype=np.uint64).astype(np.uint32)
    sw = rng.uniform(0.01, 0.05, d_out).astype(np.float32)
    A = rng.integers(-127, 128, size=(r, d_in)).astype(np.int8)
    sA = np.full(r, 1e-3, dtype=np.float32)
    Bm = rng.integers(-127, 128, size=(d_out, r)).astype(np.int8)
    sB = np.full(d_out, 1e-3, dtype=np.float32)
    q = rng.integers(-127, 128, size=(B, d_in)).astype(np.int8)
    q[0, :5] = 127  # extremes in the first row
    s = rng.uniform(0.01, 0.05, B).astype(np.float32)
    acc, y = k_proj(_dev(bits), _dev(sw), _dev(A), _dev(sA), _dev(Bm), _dev(sB), _dev(q), _dev(s))
    acc, y = acc.cpu().numpy(), y.cpu().numpy()
    for b in range(B):
        yo, acco, _ = oracle.proj(bits, sw, A, sA, Bm, sB, q[b], s[b])
        assert np.array_equal(acc[b], acco), b
        assert_close(y[b], yo, what=f"y[{b}]")


def test_k_proj_all_sign_probes():
    from bit_quantized_mamba_amd import k_proj
    d_in, d_out, r = 2048, 64, 16
    rng = np.random.default_rng(3)
    bits = np.zeros((d_out, d_in // 32), dtype=np.uint32)
    bits[: d_out // 2] = 0xFFFFFFFF
    q = rng.integers(-127, 128, size=(1, d_in)).astype(np.int8)
    z = np.zeros
    acc, _ = k_proj(_dev(bits), _dev(np.ones(d_out, np.float32)), _dev(z((r, d_in), np.int8)),
                    _dev(np.ones(r, np.float32)), _dev(z((d_out, r), np.int8)), _dev(np.ones(d_out, np.float32)),
                    _dev(q), _dev(np.ones(1, np.float32)))
    acc = acc.cpu().numpy()[0]
    tot = int(q.astype(np.int64).sum())
    assert np.all(acc[: d_out // 2] == tot) and np.all(acc[d_out // 2:] == -tot)
    # one-hot probes read single bits
    bits = rng.integers(0, 2**32, size=(d_out, d_in // 32), dtype=np.uint64).astype(np.uint32)
    for j in (0, 31, 32, 1000, 2047):
        q = np.zeros((1, d_in), dtype=np.int8)
        q[0, j] = 127
        acc, _ = k_proj(_dev(bits), _dev(np.ones(d_out, np.float32)), _dev(z((r, d_in), np.int8)),
                        _dev(np.ones(r, np.float32)), _dev(z((d_out, r), np.int8)), _dev(np.ones(d_out, np.float32)),
                        _dev(q), _dev(np.ones(1, np.float32)))
        want = np.where((bits[:, j // 32] >> np.uint32(j % 32)) & 1, 127, -127)
        assert np.array_equal(acc.cpu().numpy()[0], want), j


# ---------------------------------------------------------------------------
# greedy argmax of the batched path: both ways a logits row is read
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("vocab", [1024, 1021], ids=["v1024", "v1021"])
@pytest.mark.parametrize("aligned", [True, False], ids=["aligned", "offset4"])
def test_argmax_rows_both_read_forms(vocab, aligned):
    """Next token = lowest index of each row's maximum logit, whether the row is
    read four floats at a time (a vocabulary that is a multiple of 4 from a
    16-byte aligned base) or one float at a time (an odd vocabulary, or a base
    4 bytes off), including an exact tie with a copy of the winning embedding
    row near the end of the vocabulary."""
    import dataclasses
    shape = dataclasses.replace(synth.TINY, vocab=vocab)
    seed = synth.SEED_BASE + 77
    B = 3
    eng = engine(shape, max_batch=B)
    eng.set_path("gemm")
    eng.load_synthetic(seed)
    toks = synth.gen_tokens(seed, 5, B, vocab)

    def step():
        eng.reset_state(B)
        buf = torch.empty(B * vocab + 4, dtype=torch.float32, device="cuda")
        lg = (buf[:B * vocab] if aligned else buf[1:1 + B * vocab]).view(B, vocab)
        lg, nx = eng.decode_step(_dev(toks.astype(np.int32)), logits=lg)
        return lg.cpu().numpy(), nx.cpu().numpy()

    lg, nx = step()
    assert np.array_equal(nx, np.argmax(lg, axis=1))
    # row 0's winner copied to the highest index that is neither it nor an
    # input token (the inputs stay as they were): the same logit bit for bit,
    # and the lower index wins
    a = int(nx[0])
    used = set(int(t) for t in toks)
    above = sorted(set(range(a + 1, vocab)) - used)
    if above:
        dup, winner = above[-1], a
    else:
        dup = min(set(range(a)) - used)
        winner = dup
    E, sE = eng.get_tensor(-1, "E"), eng.get_tensor(-1, "sE")
    E[dup], sE[dup] = E[a], sE[a]
    eng.set_tensor(-1, "E", E)
    eng.set_tensor(-1, "sE", sE)
    lg2, nx2 = step()
    keep = np.arange(vocab) != dup
    assert np.array_equal(lg2[:, keep], lg[:, keep])
    assert lg2[0, dup] == lg2[0, a]
    assert int(nx2[0]) == winner
    assert np.array_equal(nx2, np.argmax(lg2, axis=1))
    eng.check()
    eng.close()
