"""Helpers shared by the GPU parity tests."""
import numpy as np

import synth

# Floating outputs are compared per tensor with the relative error floored at
# the tensor's RMS:  max_i |g_i - o_i| / max(|o_i|, rms(o)) <= TOL.
TOL = 1e-3


def rel_err(gpu, ref) -> float:
    g = np.asarray(gpu, dtype=np.float64).reshape(-1)
    o = np.asarray(ref, dtype=np.float64).reshape(-1)
    if o.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    den = np.maximum(np.abs(o), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(g - o) / den))


def assert_close(gpu, ref, tol=TOL, what=""):
    e = rel_err(gpu, ref)
    assert e <= tol, f"{what}: relative error {e:.3e} > {tol:.1e}"


def token_ok(gpu_tok: int, ref_logits: np.ndarray, tol: float = 2e-3) -> bool:
    """The GPU's greedy token is accepted if the oracle ranks it within a near-tie
    band of the maximum (several tokens are correct when logits nearly tie)."""
    m = float(ref_logits.max())
    rms = float(np.sqrt(np.mean(ref_logits ** 2)))
    return float(ref_logits[gpu_tok]) >= m - tol * max(abs(m), rms)


def engine(shape, max_batch=1):
    from bit_quantized_mamba_amd import Engine
    return Engine.from_shape(shape, max_batch=max_batch)


def ssm_canonical_to_oracle(ssm_l):
    return np.ascontiguousarray(ssm_l, dtype=np.float64)


def trace_to_numpy(tr):
    return {k: v.cpu().numpy() for k, v in tr.items()}


def oracle_follow_step(om, st, tok, tr, b=0):
    """One oracle decode step of sequence b that takes the GPU's int8 codes
    (recorded in trace `tr`) wherever they are correct roundings of the
    oracle's own values -- several codes are correct near a rounding tie --
    and otherwise raises.  The oracle runs on its own residual stream.

    Returns (h per layer [L+1][d_model], logits, argmax)."""
    import oracle
    s = om.s
    h = om.embed(int(tok))
    hs = [h]
    for l in range(s.n_layer):
        h = oracle.layer_step(s, om.weights["layers"][l], h, st.conv[l], st.ssm[l],
                              q1_force=tr["q1"][l, b], q2_force=tr["q2"][l, b])
        hs.append(h)
    best, logits, _, _ = om.lm_head(h, qf_force=tr["qf"][b])
    return np.array(hs), logits, best
