"""The density-field SSM-state codec on the device against the oracle's
(gist.science technical summary §2.D): fields and scales bit-exact on the same
fp32 rows (row-major entry points and the engine's state layout), readout
bit-exact, and a decode with the codec applied at every 8-token chunk
boundary followed by the oracle, which takes the GPU's fields after checking
them against its own encoding of the GPU's state."""
import numpy as np
import pytest

import oracle
import synth
from tests._common import assert_close, engine, oracle_follow_step, trace_to_numpy

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TWO_1P3B = synth.Shape(n_layer=2, d_model=2048, d_inner=4096, d_state=128, headdim=64, vocab=1024)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _rows(rng, n, count):
    parts = [rng.standard_normal((count, n)),
             rng.uniform(-1, 1, (count, n)) * 1e-3,
             rng.standard_cauchy((count, n)),
             rng.standard_normal((count, n)) * (rng.uniform(0, 1, (count, n)) < 0.1)]
    x = np.concatenate(parts).astype(np.float32)
    x[0] = 0.0                      # all-zero row
    x[1] = 2.5                      # constant row
    x[2] = -np.float32(1e-30)       # tiny constant row
    x[3, ::2] = 1.0                 # densities exactly on the levels
    x[3, 1::2] = -1.0
    return x


@pytest.mark.parametrize("n", [16, 32, 64, 128])
def test_k_density_bit_exact(n):
    from bit_quantized_mamba_amd import k_density_decode, k_density_encode
    rng = np.random.default_rng(n)
    x = _rows(rng, n, 64)
    f, sc = k_density_encode(_dev(x))
    y = k_density_decode(f, sc)
    f, sc, y = f.cpu().numpy().view(np.uint32), sc.cpu().numpy(), y.cpu().numpy()
    for r in range(x.shape[0]):
        fo, so = oracle.density_encode(x[r])
        assert sc[r] == so, r
        assert np.array_equal(f[r], fo), r
        assert np.array_equal(y[r], oracle.density_decode(fo, so, n)), r


@pytest.mark.parametrize("shape", [synth.TINY, TWO_1P3B], ids=["tiny", "1p3b"])
def test_state_pack_unpack_roundtrip(shape):
    B = 3
    eng = engine(shape, max_batch=B)
    eng.load_synthetic(synth.SEED_BASE)
    rng = np.random.default_rng(7)
    conv = rng.standard_normal((shape.n_layer, shape.conv_dim, shape.d_conv - 1)).astype(np.float32)
    ssm = [(rng.standard_normal((shape.n_layer, shape.n_heads, shape.headdim, shape.d_state))
            * rng.uniform(0.01, 3.0)).astype(np.float32) for _ in range(B)]
    for b in range(B):
        eng.set_state(b, conv, ssm[b])
    f, sc = eng.state_pack(1, 2)
    f = f.cpu().numpy().view(np.uint32)
    sc = sc.cpu().numpy()
    want = []
    for k, b in enumerate((1, 2)):
        rows = ssm[b].reshape(-1, shape.d_state)
        fk, sk = f[k].reshape(rows.shape[0], -1), sc[k].reshape(-1)
        dec = np.empty_like(rows)
        for r in range(rows.shape[0]):
            fo, so = oracle.density_encode(rows[r])
            assert sk[r] == so and np.array_equal(fk[r], fo), (b, r)
            dec[r] = oracle.density_decode(fo, so, shape.d_state)
        want.append(dec.reshape(ssm[b].shape))
    # unpack slot 1's and slot 2's fields into slots 0 and 1
    eng.state_unpack(torch.from_numpy(f.view(np.int32)).cuda(), torch.from_numpy(sc).cuda(), seq0=0)
    assert np.array_equal(eng.get_state(0)[1], want[0]) and np.array_equal(eng.get_state(1)[1], want[1])
    assert np.array_equal(eng.get_state(0)[0], conv)  # the conv state is untouched
    # the in-place round trip equals unpack(pack)
    eng.set_state(2, conv, ssm[2])
    eng.state_roundtrip(2, 1)
    assert np.array_equal(eng.get_state(2)[1], want[1])
    eng.check()
    eng.close()


@pytest.mark.parametrize("shape,path", [(synth.TINY, "persistent"), (synth.TINY, "gemm"), (TWO_1P3B, "persistent")],
                         ids=["tiny-persistent", "tiny-gemm", "1p3b-persistent"])
def test_decode_with_codec_at_chunk_boundaries_follows_oracle(shape, path):
    # 6 chunks of 8 greedy tokens; at each boundary the GPU packs its state,
    # the fields must equal the oracle's encoding of the GPU's own state (the
    # same fp32 rows), then both continue from the fields' readout
    seed = synth.SEED_BASE + 51
    eng = engine(shape)
    eng.set_path(path)
    eng.load_synthetic(seed)
    om = oracle.Model(shape, synth.gen_model(shape, seed))
    st = oracle.State(shape)
    tok = int(synth.gen_tokens(seed, 2, 1, shape.vocab)[0])
    for chunk in range(6):
        for step in range(8):
            tr = trace_to_numpy(eng.trace_step(_i32([tok])))
            _, ol, _ = oracle_follow_step(om, st, tok, tr)
            assert_close(tr["logits"][0], ol, what=f"logits chunk {chunk} step {step}")
            tok = int(np.argmax(tr["logits"][0]))
        conv_g, ssm_g = eng.get_state(0)
        assert_close(ssm_g, st.ssm, what=f"ssm state before boundary {chunk}")
        f, sc = eng.state_pack(0, 1)
        f = f.cpu().numpy().view(np.uint32)[0].reshape(-1, shape.d_state // 8)
        sc = sc.cpu().numpy()[0].reshape(-1)
        rows = ssm_g.reshape(-1, shape.d_state)
        dec = np.empty_like(rows)
        for r in range(rows.shape[0]):
            fo, so = oracle.density_encode(rows[r])
            assert sc[r] == so and np.array_equal(f[r], fo), (chunk, r)
            dec[r] = oracle.density_decode(fo, so, shape.d_state)
        eng.state_roundtrip(0, 1)
        assert np.array_equal(eng.get_state(0)[1], dec.reshape(ssm_g.shape))
        st.ssm[:] = dec.reshape(ssm_g.shape).astype(np.float64)
    eng.check()
    eng.close()
