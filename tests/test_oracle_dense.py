"""A second, dense statement of the decode step in NumPy fp64, written from
the readings of the pages (gist.science technical summary §2.B and §2.C: a
1-bit sign scaffold with an int8 rank-16 LoRA on in_proj and out_proj, int8
per-row-scaled tied embedding / LM head, the conv shift register and the SSM
recurrence of the Mamba-2 block), used to pin the oracle's composition of
its stage functions.  Nothing here calls the oracle's stage functions: the
scaffold is unpacked to a dense +-1 matrix, every projection is a library
matrix product, the conv is a window dot product, the SSM state update is
one broadcast expression.  Agreement to 1e-12 over several decode steps (and
on the 1.3B-shaped layer) rules out a dropped term, a wrong sign, a wrong
split position or a transposed operand in the oracle.  CPU only."""
import numpy as np
import pytest

import oracle
import synth

EPS = 1e-5


def _unpack_signs(bits):
    """uint32 [d_out][d_in/32], bit k of word j = input 32 j + k, set -> +1."""
    d_out = bits.shape[0]
    b = np.unpackbits(np.ascontiguousarray(bits).view(np.uint8), bitorder="little").reshape(d_out, -1)
    return np.where(b == 1, 1, -1).astype(np.int64)


def _quant(u):
    """Per-token symmetric absmax int8, decided in fp32 (value rounded to fp32
    once; 127 / amax one fp32 division; product and rounding in fp32, ties to
    even; clamp to [-127, 127]); an all-zero vector gives zero codes, scale 0."""
    uf = np.asarray(u, dtype=np.float64).astype(np.float32)
    amax = np.float32(np.max(np.abs(uf))) if uf.size else np.float32(0)
    if amax == 0:
        return np.zeros(uf.size, np.int64), 0.0
    inv = np.float32(127.0) / amax
    q = np.clip(np.rint(uf * inv), -127, 127).astype(np.int64)
    return q, float(amax / np.float32(127.0))


def _rmsnorm(x, w):
    return x / np.sqrt(np.mean(x * x) + EPS) * w.astype(np.float64)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def _softplus(a):
    return np.logaddexp(0.0, a)


class Dense:
    def __init__(self, s, weights):
        self.s = s
        self.L = []
        for lay in weights["layers"]:
            d = dict(lay)
            d["Win"] = _unpack_signs(lay["in_bits"])
            d["Wout"] = _unpack_signs(lay["out_bits"])
            self.L.append(d)
        self.E = weights["E"].astype(np.int64)
        self.sE = weights["sE"].astype(np.float64)
        self.fn = weights["final_norm"]

    @staticmethod
    def _proj(W, sw, A, sA, Bm, sB, q, s):
        acc = W @ q
        t = (A.astype(np.int64) @ q).astype(np.float64) * sA.astype(np.float64) * s
        return acc * sw.astype(np.float64) * s + sB.astype(np.float64) * (Bm.astype(np.float64) @ t), acc

    def layer(self, l, h, conv, ssm):
        s, d = self.s, self.L[l]
        di, N, H, P = s.d_inner, s.d_state, s.n_heads, s.headdim
        q1, s1 = _quant(_rmsnorm(h, d["norm_w"]))
        zx, acc1 = self._proj(d["Win"], d["in_sw"], d["in_A"], d["in_sA"], d["in_B"], d["in_sB"], q1, s1)
        z, xbc, dt_raw = zx[:di], zx[di:di + s.conv_dim], zx[di + s.conv_dim:]
        win = np.concatenate([conv, xbc[:, None]], axis=1)           # [C][K], oldest first
        xc = _silu(d["conv_b"].astype(np.float64) + np.sum(d["conv_w"].astype(np.float64) * win, axis=1))
        conv[:] = win[:, 1:]
        x = xc[:di].reshape(H, P)
        Bv, Cv = xc[di:di + N], xc[di + N:di + 2 * N]
        dt = _softplus(dt_raw + d["dt_bias"].astype(np.float64))
        dA = np.exp(-dt * np.exp(d["A_log"].astype(np.float64)))
        ssm[:] = ssm * dA[:, None, None] + (dt[:, None] * x)[:, :, None] * Bv[None, None, :]
        y = ssm @ Cv + d["D"].astype(np.float64)[:, None] * x
        g = y.reshape(-1) * _silu(z)
        q2, s2 = _quant(_rmsnorm(g, d["gnorm_w"]))
        out, acc2 = self._proj(d["Wout"], d["out_sw"], d["out_A"], d["out_sA"], d["out_B"], d["out_sB"], q2, s2)
        return h + out, (q1, q2, acc1, acc2)

    def step(self, tok, conv, ssm):
        h = self.E[tok].astype(np.float64) * self.sE[tok]
        for l in range(self.s.n_layer):
            h, _ = self.layer(l, h, conv[l], ssm[l])
        qf, sf = _quant(_rmsnorm(h, self.fn))
        logits = (self.E @ qf).astype(np.float64) * self.sE * sf
        return logits, h


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def test_dense_restatement_matches_oracle_decode():
    # the 2-layer test stack: 8 greedy decode steps, state carried
    s = synth.TINY
    seed = synth.SEED_BASE + 21
    w = synth.gen_model(s, seed)
    om = oracle.Model(s, w)
    dn = Dense(s, w)
    st = oracle.State(s)
    conv = np.zeros_like(st.conv)
    ssm = np.zeros_like(st.ssm)
    tok = int(synth.gen_tokens(seed, 0, 1, s.vocab)[0])
    for step in range(8):
        nxt, lo, trace = om.decode_step(st, tok, want_trace=True)
        ld, hd = dn.step(tok, conv, ssm)
        assert _rel(ld, lo) <= 1e-12, (step, _rel(ld, lo))
        assert _rel(hd, trace[-1]) <= 1e-12, step
        assert _rel(ssm, st.ssm) <= 1e-12 and _rel(conv, st.conv) <= 1e-12, step
        assert int(np.argmax(ld)) == nxt, step
        tok = nxt


@pytest.mark.parametrize("steps", [3])
def test_dense_restatement_matches_oracle_1p3b_layer(steps):
    # one layer at the 1.3B shape (headdim 64, d_state 128, 8512 in_proj rows):
    # the split positions, head/channel strides and B/C sharing at full size
    s = synth.LAYER_1P3B
    seed = synth.SEED_BASE + 22
    lay = synth.gen_layer(s, seed, 0)
    dn = Dense(s, {"layers": [lay], "E": np.zeros((1, s.d_model), np.int8), "sE": np.zeros(1, np.float32),
                   "final_norm": np.ones(s.d_model, np.float32)})
    cs = np.zeros((s.conv_dim, s.d_conv - 1))
    ss = np.zeros((s.n_heads, s.headdim, s.d_state))
    cd, sd = cs.copy(), ss.copy()
    for t in range(steps):
        h = synth.gen_fp16_normal(seed, 1, s.d_model, start=t * s.d_model).astype(np.float64)
        ho, dbg = oracle.layer_step(s, lay, h, cs, ss, want_dbg=True)
        hd, (q1, q2, acc1, acc2) = dn.layer(0, h, cd, sd)
        assert np.array_equal(q1, dbg["q1"]) and np.array_equal(q2, dbg["q2"]), t
        # the oracle's exact scaffold sums on the same codes
        assert np.array_equal(acc1, oracle.scaffold_acc(lay["in_bits"], dbg["q1"])), t
        assert np.array_equal(acc2, oracle.scaffold_acc(lay["out_bits"], dbg["q2"])), t
        assert _rel(hd - h, ho - h) <= 1e-12, t
        assert _rel(sd, ss) <= 1e-12 and _rel(cd, cs) <= 1e-12, t


def test_dense_restatement_detects_planted_mistakes():
    # The comparison above would catch the mistakes it is meant to catch:
    # each planted change to the dense statement moves its result by far
    # more than 1e-12 on the same inputs.
    s = synth.TINY
    seed = synth.SEED_BASE + 23
    w = synth.gen_model(s, seed)
    base = Dense(s, w)
    tok = 5

    def run(d):
        conv = np.zeros((s.n_layer, s.conv_dim, s.d_conv - 1))
        ssm = np.zeros((s.n_layer, s.n_heads, s.headdim, s.d_state))
        for _ in range(3):
            lg, _ = d.step(tok, conv, ssm)
        return lg

    ref = run(base)
    planted = []
    d = Dense(s, w)
    d.L[0]["Win"] = -d.L[0]["Win"]                       # sign convention of the scaffold bits
    planted.append(d)
    d = Dense(s, w)
    d.L[1]["conv_w"] = d.L[1]["conv_w"][:, ::-1].copy()   # conv taps in the wrong order
    planted.append(d)
    d = Dense(s, w)
    d.L[0]["in_B"] = np.zeros_like(d.L[0]["in_B"])       # the LoRA term dropped
    planted.append(d)
    for i, p in enumerate(planted):
        assert _rel(run(p), ref) > 1e-6, i
