"""GPU parity of sampling-mode verification (mk_lmhead_sample): the top-k
candidates of every row against the oracle's float64 logits, their logit
values, and the accept / resample decisions against the oracle's sampler
run on the GPU's own candidates (teacher-forced), on the same uniforms."""
import numpy as np
import pytest

import oracle
import synth
from synth import recipes
from tests._util import need_gpu, say, to_dev, to_np

pytestmark = pytest.mark.gpu

MARGIN = 1e-5  # decisions this close to their boundary may go either way (fp32 vs float64)


def _mk():
    import bit_weight_streaming_q4_amd as mk
    return mk


def _u(x):
    """fp32 uniforms in [0, 1) (the float64 draws rounded down into range)."""
    return np.minimum(np.asarray(x, np.float64).astype(np.float32), np.float32(1.0 - 2.0 ** -24))


def _run(mk, torch, Wd, hid, gs, drafts, k, tau, ua, us, V=None):
    T = hid.shape[0]
    G = 1 if gs is None else len(gs) - 1
    ti = torch.empty(T, 32, dtype=torch.int32, device="cuda")
    tv = torch.empty(T, 32, dtype=torch.float32, device="cuda")
    na = torch.empty(G, dtype=torch.int32, device="cuda")
    tok = torch.empty(T, dtype=torch.int32, device="cuda")
    dr = to_dev(np.asarray(drafts, np.int32)) if len(drafts) else None
    mk.mk_lmhead_sample(Wd, to_dev(hid), gs, dr, k, tau, to_dev(_u(ua)), to_dev(_u(us)), na, tok, topk_idx=ti,
                        topk_logit=tv, V=V)
    return to_np(ti), to_np(tv), to_np(na), to_np(tok)


def _check(W16, hid, gs, drafts, k, tau, ua, us, ti, tv, na, tok):
    T, H = hid.shape
    r = oracle.lmhead(W16, hid, return_logits=True)
    lg = r["logits"]
    # a bound on the fp32 error of any logit of the row
    wmax = np.abs(W16.view(np.float16).astype(np.float64)).max()
    bound = 8 * 2.0 ** -24 * np.sqrt(H) * np.abs(hid.astype(np.float64)).sum(1) * wmax
    oi, ov = oracle.topk_rows(lg, k)
    for t in range(T):
        got = [int(i) for i in ti[t] if i >= 0]
        ref = [int(i) for i in oi[t] if i >= 0]
        assert len(got) == len(ref) and all(i < 0 for i in ti[t, len(got):])
        if got != ref:
            # only a near-tie at the k-th boundary may swap a candidate
            srt = np.sort(lg[t][~np.isnan(lg[t])])[::-1]
            assert len(srt) > k and srt[k - 1] - srt[k] <= 2 * bound[t], (t, got, ref)
            assert len(set(got) ^ set(ref)) == 2
        if got:
            assert np.all(np.abs(tv[t, :len(got)].astype(np.float64) - lg[t, got]) <= bound[t] + 1e-30), t
    # decisions on the GPU's own candidates
    gsx = [0, T] if gs is None else list(gs)
    n_ref, t_ref, margin = oracle.sample_verify(ti, tv.astype(np.float64), gsx, drafts, tau,
                                                _u(ua).astype(np.float64), _u(us).astype(np.float64))
    for g in range(len(gsx) - 1):
        r0, r1 = gsx[g], gsx[g + 1]
        if np.min(margin[r0:r1]) <= MARGIN:
            continue
        assert na[g] == n_ref[g] and np.array_equal(tok[r0:r1], t_ref[r0:r1]), (g, na[g], n_ref[g])
    return n_ref


def _drafts(lg_top, gs, T, V, rng):
    gsx = [0, T] if gs is None else gs
    out = []
    for g in range(len(gsx) - 1):
        for i in range(gsx[g + 1] - gsx[g] - 1):
            c = rng.integers(0, 4)
            out.append(int(lg_top[gsx[g] + i]) if c < 2 else int(rng.integers(0, V)) if c == 2 else -7)
    return np.asarray(out, np.int32)


@pytest.mark.parametrize("T,gs", [(5, None), (12, [0, 3, 6, 9, 12]), (16, [0, 5, 6, 16]), (1, None)])
def test_sample_small_vs_oracle(T, gs):
    torch = need_gpu()
    mk = _mk()
    V, H = 1000, 512
    W = synth.normal_f16(6, 10, 0, V * H, 0.0, 0.02).reshape(V, H)
    Wd = to_dev(W)
    rng = np.random.default_rng(T)
    for k, tau in ((32, 0.6), (8, 1.0), (1, 0.6), (20, 0.05)):
        for trial in range(3):
            hid = synth.normal_f32(6, 11 + trial, T, T * H).reshape(T, H)
            top1 = oracle.lmhead(W, hid)["top1"]
            drafts = _drafts(top1, gs, T, V, rng)
            ua = synth.uniform_f64(6, 12, 100 * T + trial, T)
            us = synth.uniform_f64(6, 13, 100 * T + trial, T)
            say("sample small", T, k, tau, trial)
            out = _run(mk, torch, Wd, hid, gs, drafts, k, tau, ua, us)
            _check(W, hid, gs, drafts, k, tau, ua, us, *out)


def test_sample_top1_equals_greedy_and_nan_rows():
    torch = need_gpu()
    mk = _mk()
    V, H, T = 1000, 512, 6
    W = synth.normal_f16(6, 20, 0, V * H, 0.0, 0.02).reshape(V, H)
    Wd = to_dev(W)
    hid = synth.normal_f32(6, 21, 0, T * H).reshape(T, H)
    gs = [0, 3, 6]
    top1 = oracle.lmhead(W, hid)["top1"]
    drafts = np.array([top1[0], top1[1], top1[3], 5], np.int32)
    # top_k = 1: every target is one-hot on the argmax, whatever the uniforms
    am = torch.empty(T, dtype=torch.int32, device="cuda")
    ng = torch.empty(2, dtype=torch.int32, device="cuda")
    tg = torch.empty(T, dtype=torch.int32, device="cuda")
    mk.mk_lmhead_verify(Wd, to_dev(hid), gs, to_dev(drafts), am, ng, tg)
    for seed in range(4):
        ua, us = synth.uniform_f64(6, 22, seed, T), synth.uniform_f64(6, 23, seed, T)
        _, _, na, tok = _run(mk, torch, Wd, hid, gs, drafts, 1, 0.6, ua, us)
        assert np.array_equal(na, to_np(ng)) and np.array_equal(tok, to_np(tg))
    # an all-NaN hidden row has no candidates: it rejects its draft and emits -1
    h = hid.copy()
    h[1] = np.nan
    ua, us = np.zeros(T), np.full(T, 0.5)
    ti, tv, na, tok = _run(mk, torch, Wd, h, gs, drafts, 8, 0.6, ua, us)
    assert (ti[1] == -1).all() and np.isneginf(tv[1]).all()
    assert na[0] == 1 and tok[0] == drafts[0] and tok[1] == -1 and tok[2] == -1


def test_sample_emitted_tokens_follow_the_target():
    """Chi-square of the first emitted token over many calls with fresh
    uniforms: it follows the row's target p, whatever the draft."""
    torch = need_gpu()
    mk = _mk()
    V, H, T = 400, 512, 3
    W = synth.normal_f16(6, 30, 0, V * H, 0.0, 0.02).reshape(V, H)
    Wd = to_dev(W)
    hid = synth.normal_f32(6, 31, 0, T * H).reshape(T, H) * 2.0  # p between 0.05 and 0.42
    k, tau = 8, 0.6
    ti, tv, _, _ = _run(mk, torch, Wd, hid, None, [0, 0], k, tau, np.zeros(T), np.zeros(T))
    assert (ti[0, :k] >= 0).all() and (ti[0, k:] == -1).all()
    w = oracle.sample_weights(tv[0, :k].astype(np.float64), tau)
    p = w / w.sum()
    d0 = int(ti[0][np.argsort(p)[-2]])  # the second most likely candidate as the draft
    n = 3000
    ua = synth.uniform_f64(6, 32, 0, n * T).reshape(n, T)
    us = synth.uniform_f64(6, 33, 0, n * T).reshape(n, T)
    counts = {}
    say("sample chi-square", n)
    for i in range(n):
        _, _, _, tok = _run(mk, torch, Wd, hid, None, [d0, 1], k, tau, ua[i], us[i])
        counts[int(tok[0])] = counts.get(int(tok[0]), 0) + 1
    obs = np.array([counts.get(int(v), 0) for v in ti[0, :k]], np.float64)
    say("candidates", ti[0, :k], "p", p, "observed", obs)
    assert obs.sum() == n
    chi2 = float((((obs - n * p) ** 2) / (n * p)).sum())
    assert chi2 < 24.3, chi2  # 7 dof, p = 0.001


def test_sample_full_vocab_twelve_rows():
    """The lm_head workload's shapes: fp16 151936 x 5120, T = 12 in 4 groups
    of 3, top_k = 32, temperature 0.6, plus the 32768-row draft-vocab prefix."""
    torch = need_gpu()
    mk = _mk()
    W = recipes.lm_head_weight()
    Wd = to_dev(W)
    gs = [0, 3, 6, 9, 12]
    rng = np.random.default_rng(7)
    for trial, V in ((0, recipes.VOCAB), (1, recipes.DRAFT_VOCAB)):
        hid = recipes.lm_hidden(12, trial=20 + trial)
        Wv = W[:V]
        top1 = oracle.lmhead(Wv, hid)["top1"]
        drafts = _drafts(top1, gs, 12, V, rng)
        ua = synth.uniform_f64(6, 40, trial, 12)
        us = synth.uniform_f64(6, 41, trial, 12)
        say("sample full", V)
        out = _run(mk, torch, Wd, hid, gs, drafts, 32, 0.6, ua, us, V=V)
        _check(Wv, hid, gs, drafts, 32, 0.6, ua, us, *out)
