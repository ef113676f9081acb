"""GPU parity of the Gated DeltaNet step with rollback: outputs and the
committed state against the oracle (which recomputes the accepted prefix
instead of replaying a ring), and chain equivalence on the GPU itself."""
import numpy as np
import pytest

import oracle
import synth
from synth import recipes
from tests._util import FP32_TOL, need_gpu, rel_err, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _mk():
    import bit_weight_streaming_q4_amd as mk
    return mk


def _inputs_dev(inp):
    return [to_dev(inp[k]) for k in ("q", "k", "v", "g", "beta")]


def _run_steps(mk, torch, S0, steps, T, accepts, nh, T_max=5):
    st = mk.DeltaNetState(nh, T_max, S=to_dev(S0.reshape(nh, 128, 128)))
    outs = []
    for s in range(steps):
        inp = steps_inputs(s, T, nh)
        q, k, v, g, b = _inputs_dev(inp)
        o = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
        mk.mk_deltanet_step(st, q, k, v, g, b, o, use_prev_acc=s > 0)
        st.n_acc[0] = int(accepts[s])
        outs.append(to_np(o))
    mk.mk_deltanet_commit(st)
    return to_np(st.S), outs


def steps_inputs(s, T, nh):
    return synth.gdn_step_inputs(4, 500 + s, T, nh, 128, 128)


# T = 5 rows per step (the workload's), the largest ring (16 rows per step,
# up to 15 replayed), two rows on a 16-row ring, and one row (nothing to
# replay).
@pytest.mark.parametrize("nh,T,T_max,steps", [(24, 5, 5, 40), (8, 16, 16, 12), (8, 2, 16, 20), (8, 1, 2, 10)])
def test_gdn_many_steps_vs_oracle(nh, T, T_max, steps):
    torch = need_gpu()
    mk = _mk()
    S0 = synth.normal_f32(4, 7, 0, nh * 128 * 128, 0.0, 0.01).reshape(nh, 128, 128)
    accepts = synth.uniform_i32(4, 8, 0, steps, 0, T - 1)
    say("gdn", nh, T, T_max, steps)
    Sg, outs = _run_steps(mk, torch, S0, steps, T, accepts, nh, T_max)
    S = S0.copy()
    for s in range(steps):
        inp = steps_inputs(s, T, nh)
        S, o = oracle.gdn_step(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], int(accepts[s]))
        assert rel_err(outs[s], o) <= FP32_TOL, (s, rel_err(outs[s], o))
    assert rel_err(Sg, S) <= FP32_TOL, rel_err(Sg, S)


def test_gdn_chain_equivalence_bit_exact():
    """Accepting every draft (a = T - 1) each step gives, bit for bit, the
    same outputs and state as feeding the same rows as T = 1 steps."""
    torch = need_gpu()
    mk = _mk()
    nh, T, steps = 16, 5, 6
    S0 = synth.normal_f32(4, 9, 0, nh * 128 * 128, 0.0, 0.01).reshape(nh, 128, 128)
    say("gdn chain")
    Sa, outs = _run_steps(mk, torch, S0, steps, T, [T - 1] * steps, nh)
    st = mk.DeltaNetState(nh, 5, S=to_dev(S0))
    for s in range(steps):
        inp = steps_inputs(s, T, nh)
        for t in range(T):
            q, k, v, g, b = (to_dev(np.ascontiguousarray(inp[n][t:t + 1])) for n in ("q", "k", "v", "g", "beta"))
            o = torch.empty(1, nh, 128, dtype=torch.float32, device="cuda")
            mk.mk_deltanet_step(st, q, k, v, g, b, o, use_prev_acc=False)
            assert np.array_equal(to_np(o)[0], outs[s][t]), (s, t)
    assert np.array_equal(to_np(st.S), Sa)


def test_gdn_full_size_256_steps():
    """The Gated DeltaNet workload as defined: 48 layers x 32 heads of 128 x
    128 fp32 state ~ N(0, .01), T = 5 rows per step, seeded accept lengths in
    0..4, 256 steps.  The GPU runs every head of every step; the oracle
    follows every 8th head (192 of 1536) through all 256 steps: their outputs
    at every step and their committed state at the end."""
    torch = need_gpu()
    mk = _mk()
    nh, T, steps = 48 * 32, 5, 256
    heads = np.arange(0, nh, 8)
    S0 = recipes.gdn_initial_state().reshape(nh, 128, 128)
    accepts = recipes.gdn_accept_lengths(steps)
    st = mk.DeltaNetState(nh, 5, S=to_dev(S0))
    S = S0[heads].copy()
    o = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
    worst = 0.0
    for s in range(steps):
        inp = recipes.gdn_step(s, T)
        q, k, v, g, b = _inputs_dev(inp)
        if s % 32 == 0:
            say("gdn 256 steps: step", s, "worst so far", worst)
        mk.mk_deltanet_step(st, q, k, v, g, b, o, use_prev_acc=s > 0)
        st.n_acc[0] = int(accepts[s])
        sub = {n: np.ascontiguousarray(inp[n][:, heads]) for n in ("q", "k", "v", "g", "beta")}
        S, oref = oracle.gdn_step(S, sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], int(accepts[s]))
        e = rel_err(to_np(o)[:, heads], oref)
        worst = max(worst, e)
        assert e <= FP32_TOL, (s, e)
    mk.mk_deltanet_commit(st)
    assert mk.mk_deltanet_status(st) == mk.MK_OK
    e = rel_err(to_np(st.S)[heads], S)
    say("gdn 256 steps: outputs worst", worst, "committed state", e)
    assert e <= FP32_TOL, e


def test_gdn_accept_length_out_of_range_is_reported():
    """An accept length outside 0..T_max-1 in the state replays nothing and
    is reported by mk_deltanet_status (then cleared)."""
    torch = need_gpu()
    mk = _mk()
    nh, T = 4, 5
    S0 = synth.normal_f32(4, 11, 0, nh * 128 * 128, 0.0, 0.01).reshape(nh, 128, 128)
    ref = mk.DeltaNetState(nh, 5, S=to_dev(S0.copy()))
    bad = mk.DeltaNetState(nh, 5, S=to_dev(S0.copy()))
    for st, acc in ((ref, 0), (bad, 7)):
        for s in range(2):
            inp = steps_inputs(s, T, nh)
            q, k, v, g, b = _inputs_dev(inp)
            o = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
            mk.mk_deltanet_step(st, q, k, v, g, b, o, use_prev_acc=s > 0)
            st.n_acc[0] = acc
    assert mk.mk_deltanet_status(ref) == mk.MK_OK
    assert mk.mk_deltanet_status(bad) == mk.MK_ERR_RANGE
    assert mk.mk_deltanet_status(bad) == mk.MK_OK  # cleared by the read
    assert np.array_equal(to_np(bad.S), to_np(ref.S))  # the bad step replayed nothing
    mk.mk_deltanet_commit(bad)  # n_acc[0] = 7 again: nothing replayed, reported
    assert mk.mk_deltanet_status(bad) == mk.MK_ERR_RANGE
    assert np.array_equal(to_np(bad.S), to_np(ref.S))
