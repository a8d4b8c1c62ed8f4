"""The seeded input generator: pinned to the published SplitMix64 outputs and
checked for the properties the workloads rely on."""
import json
import os

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_splitmix64_published_outputs():
    g = json.load(open(os.path.join(HERE, "golden", "splitmix64.json")))
    st = g["state"]
    want = [int(x) for x in g["outputs"]]
    got_scalar = [synth.mix64_int((st + k * synth.GAMMA) % (1 << 64)) for k in range(len(want))]
    assert got_scalar == want
    xs = np.array([(st + k * synth.GAMMA) % (1 << 64) for k in range(len(want))], dtype=np.uint64)
    assert [int(v) for v in synth.mix64(xs)] == want


def test_draws_are_position_pure():
    # any slice of a stream equals the same slice of the whole stream
    full = synth.draws(7, 3, 0, 1000)
    part = synth.draws(7, 3, 400, 100)
    assert np.array_equal(full[400:500], part)
    # distinct tids / seeds give distinct streams
    assert not np.array_equal(full, synth.draws(7, 4, 0, 1000))
    assert not np.array_equal(full, synth.draws(8, 3, 0, 1000))


def test_draw_definition_scalar():
    seed, tid = 0xDF55, 14
    key = synth.mix64_int(seed ^ (tid << 32))
    for i in (0, 1, 12345):
        assert int(synth.draws(seed, tid, i, 1)[0]) == synth.mix64_int((key + i) % (1 << 64))


def test_distributions_ranges():
    u = synth.gen_uniform(1, 2, 100000, 0.01, 0.05)
    assert u.dtype == np.float32 and u.min() >= 0.01 and u.max() <= 0.05
    assert abs(float(u.mean()) - 0.03) < 1e-3
    i8 = synth.gen_int8(1, 3, 100000)
    assert i8.min() == -127 and i8.max() == 127
    w = synth.gen_words(1, 4, 20000)
    ones = np.unpackbits(w.view(np.uint8)).mean()
    assert abs(ones - 0.5) < 0.01
    n = synth.gen_normal(1, 5, 50000)
    assert abs(float(n.mean())) < 0.03 and abs(float(n.std()) - 1.0) < 0.03
    assert n.min() >= -6 and n.max() <= 6


def test_uniform_rounding_is_single_fp64_expression():
    # U(a,b) = fp32(a + (b - a) * u) in fp64 without contraction
    d = synth.draws(11, 12, 0, 64)
    u = (d >> np.uint64(40)).astype(np.float64) * 2.0 ** -24
    want = np.array([np.float32(-0.5 + 1.0 * float(x)) for x in u], dtype=np.float32)
    assert np.array_equal(synth.gen_uniform(11, 12, 64, -0.5, 0.5), want)


def test_irwin_hall_exact_sum():
    d = synth.draws(3, 9, 0, 24)
    u = (d >> np.uint64(40)).astype(np.float64) * 2.0 ** -24
    want = np.array([np.float32(sum(u[12 * i:12 * i + 12]) - 6.0) for i in range(2)], dtype=np.float32)
    assert np.array_equal(synth.gen_normal(3, 9, 2), want)


def test_layer_shapes():
    s = synth.FULL_1P3B
    assert s.d_in_proj == 8512 and s.conv_dim == 4352 and s.n_heads == 64
    t = synth.TINY
    assert t.d_in_proj == 1072 and t.conv_dim == 544 and t.n_heads == 16
    lay = synth.gen_layer(t, 5, 1)
    for k in synth.LAYER_KINDS:
        shp, dt = synth.layer_tensor_spec(t, k)
        assert lay[k].shape == shp and lay[k].dtype == dt
