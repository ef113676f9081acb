"""GPU parity of the on-device MTP draft loop (mk_mtp_draft): every pass is
checked teacher-forced against the oracle (the oracle's pass applied to the
GPU's own inputs of that pass: catch-up rows, then each group's chain with
the GPU's drafts), each draft against the oracle's argmax over the
draft-vocabulary prefix (near-tie carve-out), and the whole loop end to end."""
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


def _emitted(gs, n_acc, V, rng):
    T = gs[-1]
    tok = np.full(T, -1, np.int32)
    for g in range(len(gs) - 1):
        for i in range(n_acc[g] + 1):
            tok[gs[g] + i] = rng.integers(0, V)
    return tok


def _argmax_ok(E16, Vd, x, got):
    """got is the oracle's argmax of RMSNorm(x) over the first Vd rows, or
    its runner-up when the two are within the near-tie bound."""
    r = oracle.lmhead(E16[:Vd], oracle.rmsnorm(x[None]))
    tau = oracle.near_tie_tau(E16.shape[1], r["abs1"], r["abs2"])[0]
    if got == r["top1"][0]:
        return True, False
    return (r["top1_val"][0] - r["top2_val"][0] <= tau and got == r["top2"][0]), True


def _check(mtp, E16, Vd, hidden, tokens, gs, n_acc, nd, drafts, trace):
    T, G = gs[-1], len(gs) - 1
    worst = 0.0
    near_any = False
    for g in range(G):
        rows = list(range(gs[g], gs[g] + n_acc[g] + 1))
        ref = oracle.mtp_block(mtp, E16, tokens[rows], hidden[rows])
        e = rel_err(trace[rows], ref)
        worst = max(worst, e)
        assert e <= FP32_TOL, (g, e)
        prev = trace[rows[-1]]
        for k in range(nd):
            if k:
                row = T + (k - 1) * G + g
                ref = oracle.mtp_block(mtp, E16, [drafts[k - 1, g]], prev[None])[0]
                e = rel_err(trace[row], ref)
                worst = max(worst, e)
                assert e <= FP32_TOL, (g, k, e)
                prev = trace[row]
            ok, near = _argmax_ok(E16, Vd, prev, int(drafts[k, g]))
            near_any |= near
            assert ok, (g, k, drafts[k, g])
    # the whole loop end to end (meaningful when no draft sat on a near-tie)
    if not near_any:
        assert np.array_equal(oracle.mtp_draft(mtp, E16, Vd, hidden, tokens, gs, n_acc, nd)["drafts"], drafts)
    return worst


def _run(mk, torch, head, E16d, Vd, hidden, gs, tokens, n_acc, nd):
    T, H = hidden.shape
    G = len(gs) - 1
    drafts = torch.full((nd, G), -9, dtype=torch.int32, device="cuda")
    trace = torch.empty(T + G * (nd - 1), H, dtype=torch.float32, device="cuda")
    mk.mk_mtp_draft(head, E16d, Vd, to_dev(hidden), gs, to_dev(tokens), to_dev(np.asarray(n_acc, np.int32)), nd,
                    drafts, trace=trace)
    return to_np(drafts), to_np(trace)


@pytest.mark.parametrize("T,gs,n_acc,nd", [(5, [0, 5], [2], 4), (5, [0, 5], [0], 1), (5, [0, 5], [4], 3),
                                           (12, [0, 3, 6, 9, 12], [2, 0, 1, 2], 2),
                                           (6, [0, 1, 6], [0, 3], 3), (16, list(range(0, 17, 2)), [1, 0] * 4, 2)])
def test_mtp_small_vs_oracle(T, gs, n_acc, nd):
    torch = need_gpu()
    mk = _mk()
    H, F, V, Vd = 256, 512, 600, 300
    mtp = {"fc": synth.q4k_fields(8, 700, H, 2 * H), "gate": synth.q4k_fields(8, 701, F, H),
           "up": synth.q4k_fields(8, 702, F, H), "down": synth.q4k_fields(8, 703, H, F)}
    head = mk.MtpHead.from_fields(mtp)
    E16 = synth.normal_f16(8, 704, 0, V * H, 0.0, 0.02).reshape(V, H)
    hidden = synth.normal_f32(8, 705, T, T * H, 0.0, 2.0).reshape(T, H)
    tokens = _emitted(gs, n_acc, V, np.random.default_rng(T + nd))
    say("mtp small", T, gs, n_acc, nd)
    drafts, trace = _run(mk, torch, head, to_dev(E16), Vd, hidden, gs, tokens, n_acc, nd)
    assert ((drafts >= 0) & (drafts < Vd)).all()
    _check(mtp, E16, Vd, hidden, tokens, gs, n_acc, nd, drafts, trace)


def test_mtp_out_of_range_accept_length_gives_no_drafts():
    torch = need_gpu()
    mk = _mk()
    H, F, V, Vd, T = 256, 512, 600, 300, 6
    mtp = {"fc": synth.q4k_fields(8, 710, H, 2 * H), "gate": synth.q4k_fields(8, 711, F, H),
           "up": synth.q4k_fields(8, 712, F, H), "down": synth.q4k_fields(8, 713, H, F)}
    head = mk.MtpHead.from_fields(mtp)
    E16 = synth.normal_f16(8, 714, 0, V * H, 0.0, 0.02).reshape(V, H)
    hidden = synth.normal_f32(8, 715, 0, T * H).reshape(T, H)
    gs = [0, 3, 6]
    tokens = _emitted(gs, [1, 2], V, np.random.default_rng(3))
    drafts, _ = _run(mk, torch, head, to_dev(E16), Vd, hidden, gs, tokens, [1, 3], 3)  # group 1: 3 rows, n_acc 3
    assert (drafts[:, 1] == -1).all() and (drafts[:, 0] >= 0).all()
    ref = oracle.mtp_draft(mtp, E16, Vd, hidden[:3], tokens[:3], [0, 3], [1], 3)["drafts"][:, 0]
    assert np.array_equal(drafts[:, 0], ref)


@pytest.mark.parametrize("T,gs,n_acc,nd", [(12, [0, 3, 6, 9, 12], [2, 0, 1, 2], 2), (5, [0, 5], [3], 4)])
def test_mtp_full_size(T, gs, n_acc, nd):
    """The stack's shapes: hidden 5120, FFN 17408, fc 5120 x 10240, the fp16
    151936 x 5120 lm_head as the tied embedding, drafting over its first
    32768 rows; 4 agents x 3 rows with 2 drafts each, and one sequence of 5
    rows with 4 drafts."""
    torch = need_gpu()
    mk = _mk()
    H, Vd = recipes.HIDDEN, recipes.DRAFT_VOCAB
    mtp = recipes.mtp_weights()
    head = mk.MtpHead.from_fields(mtp)
    E16 = recipes.stack_lm_head()
    hidden = recipes.stack_step_input(50, T)
    tokens = _emitted(gs, n_acc, recipes.VOCAB, np.random.default_rng(11))
    say("mtp full", T, nd)
    drafts, trace = _run(mk, torch, head, to_dev(E16), Vd, hidden, gs, tokens, n_acc, nd)
    worst = _check(mtp, E16, Vd, hidden, tokens, gs, n_acc, nd, drafts, trace)
    say("mtp full worst", worst, "drafts", drafts.T.tolist())
