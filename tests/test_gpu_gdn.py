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


def _run_steps(mk, torch, S0, steps, T, accepts, nh):
    st = mk.DeltaNetState(nh, 5, S=to_dev(S0.reshape(nh, 128, 128)))
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


def test_gdn_many_steps_vs_oracle():
    torch = need_gpu()
    mk = _mk()
    nh, T, steps = 24, 5, 40
    S0 = synth.normal_f32(4, 7, 0, nh * 128 * 128, 0.0, 0.01).reshape(nh, 128, 128)
    accepts = synth.uniform_i32(4, 8, 0, steps, 0, T - 1)
    say("gdn", nh, T, steps)
    Sg, outs = _run_steps(mk, torch, S0, steps, T, accepts, nh)
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


def test_gdn_full_size_steps():
    """48 layers x 32 heads of 128 x 128 fp32 state ~ N(0, .01), T = 5,
    seeded accept lengths in 0..4 (first steps of the 256-step workload)."""
    torch = need_gpu()
    mk = _mk()
    nh, T, steps = 48 * 32, 5, 4
    S0 = recipes.gdn_initial_state()
    accepts = recipes.gdn_accept_lengths(steps)
    st = mk.DeltaNetState(nh, 5, S=to_dev(S0.reshape(nh, 128, 128)))
    S = S0.reshape(nh, 128, 128).copy()
    for s in range(steps):
        inp = recipes.gdn_step(s, T)
        q, k, v, g, b = _inputs_dev(inp)
        o = torch.empty(T, nh, 128, dtype=torch.float32, device="cuda")
        say("gdn full step", s)
        mk.mk_deltanet_step(st, q, k, v, g, b, o, use_prev_acc=s > 0)
        st.n_acc[0] = int(accepts[s])
        S, oref = oracle.gdn_step(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], int(accepts[s]))
        assert rel_err(to_np(o), oref) <= FP32_TOL
    mk.mk_deltanet_commit(st)
    assert rel_err(to_np(st.S), S) <= FP32_TOL
