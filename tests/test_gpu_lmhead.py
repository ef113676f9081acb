"""GPU parity of lm_head + greedy argmax + accepted-prefix verification."""
import numpy as np
import pytest

import oracle
import synth
from synth import recipes
from tests._util import need_gpu, say, to_dev, to_np

pytestmark = pytest.mark.gpu


def _mk():
    import bit_weight_streaming_q4_amd as mk
    return mk


def _run(mk, torch, W16d, hid, gs, drafts, V=None):
    T = hid.shape[0]
    G = 1 if gs is None else len(gs) - 1
    am = torch.empty(T, dtype=torch.int32, device="cuda")
    na = torch.empty(G, dtype=torch.int32, device="cuda")
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    dr = to_dev(np.asarray(drafts, np.int32)) if len(drafts) else None
    mk.mk_lmhead_verify(W16d, to_dev(hid), gs, dr, am, na, tok, V=V)
    return to_np(am), to_np(na), to_np(tok)


def _check(W16, hid, am, na, tok, gs, drafts):
    """argmax equals the oracle's except on flagged near-tie rows (where
    either of the two candidates is accepted); n_acc and tokens equal the
    oracle's verification of the GPU argmax."""
    r = oracle.lmhead(W16, hid)
    tau = oracle.near_tie_tau(W16.shape[1], r["abs1"], r["abs2"])
    near = (r["top1_val"] - r["top2_val"]) <= tau
    for t in range(hid.shape[0]):
        if near[t]:
            assert am[t] in (r["top1"][t], r["top2"][t])
        else:
            assert am[t] == r["top1"][t], (t, am[t], r["top1"][t])
    gsx = [0, hid.shape[0]] if gs is None else gs
    n_ref, tok_ref = oracle.verify(am, gsx, drafts)
    assert np.array_equal(na, n_ref)
    assert np.array_equal(tok, tok_ref)
    return r, near


def test_lmhead_small_ragged_groups_ties_nan():
    torch = need_gpu()
    mk = _mk()
    V, H = 1000, 512  # V not a multiple of 64
    W = synth.normal_f16(3, 60, 0, V * H, 0.0, 0.02).reshape(V, H)
    for T, gs in ((5, None), (12, [0, 3, 6, 9, 12]), (1, None), (16, [0, 5, 6, 16]), (2, None),
                  (8, [0, 2, 4, 6, 8]), (9, [0, 1, 9]), (16, list(range(17)))):
        hid = synth.normal_f32(3, 61, T, T * H).reshape(T, H)
        r = oracle.lmhead(W, hid)
        G = 1 if gs is None else len(gs) - 1
        gsx = [0, T] if gs is None else gs
        drafts = []
        for g in range(G):
            for i in range(gsx[g + 1] - gsx[g] - 1):
                drafts.append(r["top1"][gsx[g] + i] if (i + g) % 3 != 2 else 7)
        say("lmhead small", T, gs)
        am, na, tok = _run(mk, torch, to_dev(W), hid, gs, drafts)
        _check(W, hid, am, na, tok, gs, np.asarray(drafts, np.int32))
    # planted exact tie between rows 311 and 900 -> lowest index; NaN row never wins
    T = 3
    hid = synth.normal_f32(3, 62, 0, T * H).reshape(T, H)
    W2 = W.copy()
    W2[311] = np.sign(hid[0]).astype(np.float16).view(np.uint16)
    W2[900] = W2[311]
    W2[5] = 0x7E00
    say("lmhead planted tie")
    am, na, tok = _run(mk, torch, to_dev(W2), hid, None, [311, 3])
    assert am[0] == 311
    assert na[0] >= 1 and tok[0] == 311
    # a draft id outside [0, V) is a mismatch
    am, na, tok = _run(mk, torch, to_dev(W2), hid, None, [-5, 1 << 30])
    assert na[0] == 0 and tok[0] == am[0] and tok[1] == -1


def test_lmhead_full_vocab_and_draft_prefix():
    """fp16 151936 x 5120 ~ N(0, .02), T = 5 rows ~ N(0, 1), drafts from the
    0.7 rule on the oracle's argmax; plus the 32768-row draft-vocab prefix and
    a 12-row, 4-group step."""
    torch = need_gpu()
    mk = _mk()
    W = recipes.lm_head_weight()
    Wd = to_dev(W)
    hist = np.zeros(5, int)
    for trial in range(3):
        hid = recipes.lm_hidden(5, trial=trial)
        r = oracle.lmhead(W, hid)
        drafts = recipes.drafts_from_argmax(r["top1"][:4], recipes.VOCAB, trial=trial)
        say("lmhead full", trial)
        am, na, tok = _run(mk, torch, Wd, hid, None, drafts)
        _check(W, hid, am, na, tok, None, drafts)
        hist[na[0]] += 1
        # draft-vocab prefix
        Wp = W[:recipes.DRAFT_VOCAB]
        rp = oracle.lmhead(Wp, hid)
        say("lmhead prefix", trial)
        amp, nap, tokp = _run(mk, torch, Wd, hid, None, rp["top1"][:4], V=recipes.DRAFT_VOCAB)
        _check(Wp, hid, amp, nap, tokp, None, rp["top1"][:4])
    hid = recipes.lm_hidden(12, trial=7)
    r = oracle.lmhead(W, hid)
    gs = [0, 3, 6, 9, 12]
    drafts = np.array([r["top1"][0], r["top1"][1], r["top1"][3], 5, r["top1"][6], r["top1"][7], 9, 9], np.int32)
    say("lmhead full T=12")
    am, na, tok = _run(mk, torch, Wd, hid, gs, drafts)
    _check(W, hid, am, na, tok, gs, drafts)


def test_lmhead_all_nan_row():
    """A hidden row of NaN has no argmax (-1): it accepts no draft, and as
    the bonus row it emits -1 (same rule as the oracle)."""
    torch = need_gpu()
    mk = _mk()
    V, H = 1000, 512
    W = synth.normal_f16(3, 63, 0, V * H, 0.0, 0.02).reshape(V, H)
    hid = synth.normal_f32(3, 64, 0, 3 * H).reshape(3, H)
    r = oracle.lmhead(W, hid)
    for nan_row, drafts in ((0, [r["top1"][0], r["top1"][1]]), (2, [r["top1"][0], r["top1"][1]]),
                            (1, [r["top1"][0], -1])):
        h = hid.copy()
        h[nan_row] = np.nan
        say("lmhead NaN row", nan_row)
        am, na, tok = _run(mk, torch, to_dev(W), h, None, drafts)
        assert am[nan_row] == -1
        ro = oracle.lmhead(W, h)
        assert ro["top1"][nan_row] == -1
        _check(W, h, am, na, tok, None, np.asarray(drafts, np.int32))
        n_ref = {0: 0, 2: 2, 1: 1}[nan_row]
        assert na[0] == n_ref and tok[n_ref] == am[n_ref]


def test_lmhead_hidden_rows_at_any_scale():
    """Rows scaled by 2^-20 and 2^16 (max |x| far above fp16's 65504) give,
    bit for bit, the argmax of the unscaled rows (the per-row power-of-two
    prescale), which is the oracle's argmax outside the near-tie carve-out."""
    torch = need_gpu()
    mk = _mk()
    V, H, T = 4000, 5120, 5
    W = synth.normal_f16(3, 65, 0, V * H, 0.0, 0.02).reshape(V, H)
    Wd = to_dev(W)
    hid = synth.normal_f32(3, 66, 0, T * H).reshape(T, H)
    r = oracle.lmhead(W, hid)
    drafts = [int(r["top1"][i]) for i in range(T - 1)]
    base = _run(mk, torch, Wd, hid, None, drafts)
    _check(W, hid, *base, None, np.asarray(drafts, np.int32))
    for e in (-20, 16, -60, 100):
        hs = (hid.astype(np.float64) * 2.0 ** e).astype(np.float32)
        assert np.array_equal(hs.astype(np.float64) / 2.0 ** e, hid)  # the scaling is exact
        say("lmhead scaled 2 **", e)
        got = _run(mk, torch, Wd, hs, None, drafts)
        for a, b in zip(got, base):
            assert np.array_equal(a, b), e
